// C ABI of libfa: argument validation (host only, before any HIP call) and
// dispatch to the gfx950 kernels. The contract is documented in include/fa.h.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Largest grid any launch of this library uses, in blocks, must fit a 1-D
// grid; the per-launch row counts are far below this bound.
constexpr long long kMaxBlocks = 0x7fffffffLL;

// Scalar checks shared by forward and backward. Returns FA_OK or an error.
int check_scalars(int B, int H, int N, int d, float scale, int causal) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  // The row-sum kernel of the backward packs the fewest rows per block (8),
  // so it has the largest grid of any launch.
  const long long rows = (long long)B * H * N;
  if (rows / 8 + 1 > kMaxBlocks) return FA_ERR_INVALID_ARG;
  // One head's [N, d] slab is addressed with 32-bit byte offsets (buffer
  // resources); fp32 tensors need N * d * 4 bytes.
  if ((long long)N * d * 4 > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

bool dtype_ok(int t) { return t == FA_F32 || t == FA_F16 || t == FA_BF16; }

fa::Elem elem(int t) {
  return t == FA_F32 ? fa::Elem::F32 : (t == FA_F16 ? fa::Elem::F16 : fa::Elem::BF16);
}

int launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, float* dsum, const int* kv_len,
               int B, int H, int N, int d, float scale, int causal, void* stream, int dtype,
               int stages) {
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, dsum, kv_len, B, H, N, d, scale, causal};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = (dtype == FA_F32) ? fa::launch_bwd_f32(a, stages, s)
                                   : fa::launch_bwd_mfma(a, elem(dtype), stages, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, const int* kv_len, void* stream, int in_dtype,
           int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype)) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;

  fa::FwdArgs a{q, k, v, o, lse, kv_len, B, H, N, d, scale, causal};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = (in_dtype == FA_F32) ? fa::launch_fwd_f32(a, s)
                                      : fa::launch_fwd_mfma(a, elem(in_dtype), elem(o_dtype), s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  if (B < 0 || H < 0 || N < 0) return 0;
  return (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
           int causal, const int* kv_len, void* workspace, size_t workspace_bytes, void* stream,
           int dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < fa_bwd_workspace_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  return launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, kv_len, B, H, N, d,
                    scale, causal, stream, dtype,
                    (int)fa::BwdStage::DQ | (int)fa::BwdStage::DKDV);
}

int fa_bwd_dsum(const void* o, const void* dout, float* dsum, int B, int H, int N, int d,
                void* stream, int dtype) {
  int st = check_scalars(B, H, N, d, 1.f, 0);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!o || !dout || !dsum) return FA_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(dout) || !aligned4(dsum)) return FA_ERR_INVALID_ARG;
  return launch_bwd(nullptr, nullptr, nullptr, o, dout, nullptr, nullptr, nullptr, nullptr, dsum,
                    nullptr, B, H, N, d, 1.f, 0, stream, dtype, (int)fa::BwdStage::DSUM);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const float* dsum, void* dk, void* dv, int B, int H, int N, int d, float scale,
                int causal, const int* kv_len, void* stream, int dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !dout || !lse || !dsum || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dk) ||
      !aligned16(dv) || !aligned4(lse) || !aligned4(dsum))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  return launch_bwd(q, k, v, nullptr, dout, lse, nullptr, dk, dv, (float*)dsum, kv_len, B, H, N,
                    d, scale, causal, stream, dtype, (int)fa::BwdStage::DKDV);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, float* dsum, void* dq, int B, int H, int N, int d, float scale,
              int causal, const int* kv_len, void* stream, int dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dsum || !dq) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned4(lse) || !aligned4(dsum))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  return launch_bwd(q, k, v, o, dout, lse, dq, nullptr, nullptr, dsum, kv_len, B, H, N, d, scale,
                    causal, stream, dtype, (int)fa::BwdStage::DQ);
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success (work enqueued)";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: null or misaligned pointer, negative size, bad scale or flag";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim must be 64 or 128; dtype pair not supported";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or smaller than fa_bwd_workspace_bytes()";
    case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
    default: return "unknown fa status";
  }
}

}  // extern "C"
