// C ABI of libfa: argument validation (host only, before any HIP call) and
// dispatch to the gfx950 kernels. The contract is documented in include/fa.h.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

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
  // No launch has more than one workgroup per 8 rows (the (O, LSE) merge at
  // d = 128 has exactly that), so this bounds every grid.
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

// O in fp32 next to 16-bit inputs: the forward's fp32 output handed to the
// backward (o_dtype == FA_F32); for fp32 inputs O is fp32 anyway.
bool o_dtype_ok(int dtype, int o_dtype) { return o_dtype == dtype || o_dtype == FA_F32; }

int launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, float* dsum, const int* kv_len,
               int B, int H, int N, int d, float scale, int causal, void* stream, int dtype,
               int o_dtype, int stages, int Hkv = 0, int gsplit = 1, float* dkv_part = nullptr,
               const unsigned char* bmask = nullptr, long long bm_sb = 0, long long bm_sh = 0) {
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, dsum, kv_len, B, H, N, d, scale, causal,
                Hkv > 0 ? Hkv : H, gsplit, dkv_part, bmask, bm_sb, bm_sh};
  a.o_f32 = (o_dtype == FA_F32 && dtype != FA_F32) ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = bmask ? fa::launch_bwd_mfma_sparse(a, elem(dtype), stages, s)
                 : (dtype == FA_F32) ? fa::launch_bwd_f32(a, stages, s)
                                     : fa::launch_bwd_mfma(a, elem(dtype), stages, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}


// Key split of a key-split forward: keys per part (a multiple of the
// kernels' 64-key tile) and the number of parts that covers N.
void split_plan(int N, int num_splits, int* ksplit, int* parts) {
  int ks = (N + num_splits - 1) / num_splits;
  ks = ((ks + 63) / 64) * 64;
  if (ks < 64) ks = 64;
  *ksplit = ks;
  *parts = N > 0 ? (N + ks - 1) / ks : 1;
}

size_t split_workspace(int B, int H, int N, int d, int parts) {
  if (parts <= 1) return 0;
  return (size_t)parts * (size_t)B * H * N * (size_t)(d + 1) * sizeof(float);
}

// Workspace of the grouped backward: D for every query row, then (when the
// dK/dV stage splits each group's query heads) the fp32 partial dK and dV.
size_t dsum_bytes_aligned(int B, int H, int N) {
  return (((size_t)B * H * N * sizeof(float)) + 255) & ~(size_t)255;
}

size_t gqa_part_bytes(int B, int Hkv, int N, int d, int gsplit) {
  if (gsplit <= 1) return 0;
  return 2 * (size_t)gsplit * B * Hkv * N * (size_t)d * sizeof(float);
}

// FP8 path: element counts of its buffers and the layout of the workspace
// of fa_fwd_fp8_incoherent (regions in this order, each at a multiple of
// 256 bytes).
struct Fp8Sizes {
  size_t qk, vt, nq, nk, bh;  // codes of Q (and of K), of V^T; scale counts
  int Np;
};
Fp8Sizes fp8_sizes(int B, int H, int N, int d) {
  Fp8Sizes z;
  z.bh = (size_t)B * H;
  z.Np = ((N + 63) / 64) * 64;
  z.qk = z.bh * N * d;
  z.vt = z.bh * d * z.Np;
  z.nq = z.bh * ((N + 127) / 128);
  z.nk = z.bh * ((N + 63) / 64);
  return z;
}
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Positions of a partial step are bounded so that every sum of a position
// difference and a row index stays inside a 32-bit int.
constexpr int kMaxPos = 1 << 29;

// Scratch of fa_bwd_noalloc: the D_i array of the backward. On the host
// this name is a stand-in, not a device address; kernels get the address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS];

// Per-device address of `scratch`, looked up once per device with that
// device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(int dev, float** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
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

  fa::FwdArgs a{q, k, v, o, lse, kv_len, B, H, N, d, scale, causal, N, 0, 0, 1, N, 0, 0, H};
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
           int dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!o_dtype_ok(dtype, o_dtype)) return FA_ERR_UNSUPPORTED;
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
                    scale, causal, stream, dtype, o_dtype,
                    (int)fa::BwdStage::DQ | (int)fa::BwdStage::DKDV);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, const int* kv_len, void* stream, int dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!o_dtype_ok(dtype, o_dtype)) return FA_ERR_UNSUPPORTED;
  const long long rows = (long long)B * H * N;
  if (rows == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  if (rows > FA_NOALLOC_MAX_ROWS) return FA_ERR_TOO_LARGE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return FA_ERR_HIP;
    if ((int)sdev != dev) return FA_ERR_INVALID_ARG;
  }
  float* dsum = nullptr;
  if (scratch_address(dev, &dsum) != hipSuccess) return FA_ERR_HIP;
  return launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, dsum, kv_len, B, H, N, d, scale, causal,
                    stream, dtype, o_dtype, (int)fa::BwdStage::DQ | (int)fa::BwdStage::DKDV);
}

int fa_bwd_dsum(const void* o, const void* dout, float* dsum, int B, int H, int N, int d,
                void* stream, int dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, 1.f, 0);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!o_dtype_ok(dtype, o_dtype)) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!o || !dout || !dsum) return FA_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(dout) || !aligned4(dsum)) return FA_ERR_INVALID_ARG;
  return launch_bwd(nullptr, nullptr, nullptr, o, dout, nullptr, nullptr, nullptr, nullptr, dsum,
                    nullptr, B, H, N, d, 1.f, 0, stream, dtype, o_dtype, (int)fa::BwdStage::DSUM);
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
                    d, scale, causal, stream, dtype, FA_F32, (int)fa::BwdStage::DKDV);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, float* dsum, void* dq, int B, int H, int N, int d, float scale,
              int causal, const int* kv_len, void* stream, int dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!o_dtype_ok(dtype, o_dtype)) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dsum || !dq) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned4(lse) || !aligned4(dsum))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  return launch_bwd(q, k, v, o, dout, lse, dq, nullptr, nullptr, dsum, kv_len, B, H, N, d, scale,
                    causal, stream, dtype, o_dtype, (int)fa::BwdStage::DQ);
}

int fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int q_pos0,
                   int k_pos0, const int* kv_len, void* stream, int in_dtype) {
  int st = check_scalars(B, H, Nq, d, scale, causal);
  if (st != FA_OK) return st;
  if (Nk < 0) return FA_ERR_INVALID_ARG;
  if ((long long)Nk * d * 4 > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  if (q_pos0 <= -kMaxPos || q_pos0 >= kMaxPos || k_pos0 <= -kMaxPos || k_pos0 >= kMaxPos)
    return FA_ERR_INVALID_ARG;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * Nq == 0) return FA_OK;
  if (!q || !o_part || !lse_part) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o_part) || !aligned4(lse_part)) return FA_ERR_INVALID_ARG;
  // With no keys, k and v are never read and may be NULL.
  if (Nk > 0 && (!k || !v || !aligned16(k) || !aligned16(v))) return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;

  fa::FwdArgs a{q, k, v, o_part, lse_part, kv_len, B, H, Nq, d, scale, causal,
                Nk, q_pos0, k_pos0, 1, Nk, 0, 0, H};
  hipError_t e = fa::launch_fwd_mfma_general(a, elem(in_dtype), (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b, void* o,
             float* lse, long long rows, int d, void* stream, int o_dtype) {
  if (rows < 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!dtype_ok(o_dtype)) return FA_ERR_UNSUPPORTED;
  if (rows / 8 + 1 > kMaxBlocks) return FA_ERR_INVALID_ARG;
  if (rows == 0) return FA_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o) || !aligned4(lse_a) || !aligned4(lse_b) ||
      !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  fa::MergeArgs m{};
  m.o[0] = o_a;
  m.o[1] = o_b;
  m.lse[0] = lse_a;
  m.lse[1] = lse_b;
  m.nparts = 2;
  m.out_o = o;
  m.out_lse = lse;
  m.rows = rows;
  hipError_t e = fa::launch_merge(m, d, elem(o_dtype), (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_split_workspace_bytes(int B, int H, int N, int d, int num_splits) {
  if (B < 0 || H < 0 || N < 0 || d < 0 || num_splits < 1 || num_splits > fa::kMaxMergeParts) return 0;
  int ks, parts;
  split_plan(N, num_splits, &ks, &parts);
  return split_workspace(B, H, N, d, parts);
}

int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, const int* kv_len, int num_splits,
                 void* workspace, size_t workspace_bytes, void* stream, int in_dtype,
                 int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (num_splits < 1 || num_splits > fa::kMaxMergeParts) return FA_ERR_INVALID_ARG;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  int ks, parts;
  split_plan(N, num_splits, &ks, &parts);
  hipStream_t s = (hipStream_t)stream;
  if (parts == 1) {
    fa::FwdArgs a{q, k, v, o, lse, kv_len, B, H, N, d, scale, causal, N, 0, 0, 1, N, 0, 0, H};
    hipError_t e = fa::launch_fwd_mfma(a, elem(in_dtype), elem(o_dtype), s);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  if (!workspace || !aligned16(workspace) || workspace_bytes < split_workspace(B, H, N, d, parts))
    return FA_ERR_WORKSPACE;
  float* wo = (float*)workspace;
  const long long so = (long long)B * H * N * d;
  const long long sl = (long long)B * H * N;
  float* wl = wo + parts * so;
  fa::FwdArgs a{q, k, v, wo, wl, kv_len, B, H, N, d, scale, causal, N, 0, 0, parts, ks, so, sl, H};
  hipError_t e = fa::launch_fwd_mfma_general(a, elem(in_dtype), s);
  if (e != hipSuccess) return FA_ERR_HIP;
  fa::MergeArgs m{};
  for (int p = 0; p < parts; ++p) {
    m.o[p] = wo + p * so;
    m.lse[p] = wl + p * sl;
  }
  m.nparts = parts;
  m.out_o = o;
  m.out_lse = lse;
  m.rows = sl;
  e = fa::launch_merge(m, d, elem(o_dtype), s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int N, int d, float scale, int causal, const int* kv_len, void* stream,
               int in_dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (Hkv < 1 || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, kv_len, B, H, N, d, scale, causal, N, 0, 0, 1, N, 0, 0, Hkv};
  hipError_t e = fa::launch_fwd_mfma(a, elem(in_dtype), elem(o_dtype), (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d) {
  if (B < 0 || H < 0 || N < 0 || Hkv < 1 || H % Hkv != 0 || (d != 64 && d != 128)) return 0;
  if (H == 0) return 0;
  return dsum_bytes_aligned(B, H, N) +
         gqa_part_bytes(B, Hkv, N, d, fa::bwd_group_split(B, H, Hkv, N, d));
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
               float scale, int causal, const int* kv_len, void* workspace,
               size_t workspace_bytes, void* stream, int dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (Hkv < 1 || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!o_dtype_ok(dtype, o_dtype)) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < fa_bwd_gqa_workspace_bytes(B, H, Hkv, N, d))
    return FA_ERR_WORKSPACE;
  const int gsplit = fa::bwd_group_split(B, H, Hkv, N, d);
  float* part = gsplit > 1 ? (float*)((char*)workspace + dsum_bytes_aligned(B, H, N)) : nullptr;
  return launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, kv_len, B, H, N, d,
                    scale, causal, stream, dtype, o_dtype,
                    (int)fa::BwdStage::DQ | (int)fa::BwdStage::DKDV, Hkv, gsplit, part);
}

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, int d, float scale, int causal, const int* kv_len,
                  const unsigned char* block_mask, long long mask_stride_b,
                  long long mask_stride_h, void* stream, int in_dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  // a mask row or column must fit the kernels' LDS list of kept blocks
  if ((N + fa::kMaskBlock - 1) / fa::kMaskBlock > fa::kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  if (mask_stride_b < 0 || mask_stride_h < 0) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  if (!block_mask) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, kv_len, B, H, N, d, scale, causal, N, 0, 0, 1, N, 0, 0, H,
                block_mask, mask_stride_b, mask_stride_h};
  hipError_t e = fa::launch_fwd_mfma_sparse(a, elem(in_dtype), elem(o_dtype), (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                  float scale, int causal, const int* kv_len, const unsigned char* block_mask,
                  long long mask_stride_b, long long mask_stride_h, void* workspace,
                  size_t workspace_bytes, void* stream, int dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!o_dtype_ok(dtype, o_dtype)) return FA_ERR_UNSUPPORTED;
  // a mask row or column must fit the kernels' LDS list of kept blocks
  if ((N + fa::kMaskBlock - 1) / fa::kMaskBlock > fa::kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  if (mask_stride_b < 0 || mask_stride_h < 0) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  if (!block_mask) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < fa_bwd_workspace_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  return launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, kv_len, B, H, N, d,
                    scale, causal, stream, dtype, o_dtype,
                    (int)fa::BwdStage::DQ | (int)fa::BwdStage::DKDV, H, 1, nullptr, block_mask,
                    mask_stride_b, mask_stride_h);
}

// Plan of the block-sparse entry points by pieces: counts[8] = {column
// items, cut columns, column slots, row items, cut rows, row slots, 0, 0};
// plan = column items, cut columns, row items, cut rows, 4 ints each.
namespace {
struct SparseItem { int bh, blk, first, slot, size; };

// Items of one kind (columns: the query blocks of key block j; rows: the
// key blocks of query block i) and the cut lines, longest pieces first.
void sparse_pieces(const unsigned char* host_mask, long long sb, long long sh, int B, int H, int nb,
                   int causal, bool columns, std::vector<SparseItem>& its, std::vector<int>& cut,
                   int* slots) {
  const int C = fa::kSparsePiece;
  *slots = 0;
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const unsigned char* m = host_mask + b * sb + h * sh;
      for (int x = 0; x < nb; ++x) {
        int n = 0;
        if (columns) {  // key block x: query blocks from the diagonal on when causal
          for (int qb = causal ? x : 0; qb < nb; ++qb) n += m[(long long)qb * nb + x] != 0;
        } else {        // query block x: key blocks up to the diagonal when causal
          for (int kb = 0; kb <= (causal ? x : nb - 1); ++kb) n += m[(long long)x * nb + kb] != 0;
        }
        const int bh = b * H + h;
        if (n <= C) {
          its.push_back({bh, x, 0, -1, n});
          continue;
        }
        const int pieces = (n + C - 1) / C;
        for (int i = 0; i < pieces; ++i)
          its.push_back({bh, x, i * C, *slots + i, std::min(C, n - i * C)});
        cut.insert(cut.end(), {bh, x, *slots, pieces});
        *slots += pieces;
      }
    }
  }
  std::stable_sort(its.begin(), its.end(),
                   [](const SparseItem& p, const SparseItem& q) { return p.size > q.size; });
  // Workgroup i runs on XCD i % 8: deal the items so that every item of head
  // bh sits at a position of class bh % 8, and the head's tiles share one
  // L2, keeping longest first within a class; once a class runs out, its
  // positions take items of the class with the most left.
  std::vector<SparseItem> cls[8];
  for (const auto& it : its) cls[it.bh % 8].push_back(it);
  size_t pos[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (size_t p = 0; p < its.size(); ++p) {
    int x = (int)(p % 8);
    if (pos[x] == cls[x].size()) {
      for (int y = 0; y < 8; ++y)
        if (cls[y].size() - pos[y] > cls[x].size() - pos[x]) x = y;
    }
    its[p] = cls[x][pos[x]++];
  }
}

// Host checks shared by the planned entry points; plan offsets in ints.
int check_plan(int B, int H, int N, const int* plan, const int* counts) {
  if (!counts) return FA_ERR_INVALID_ARG;
  for (int i = 0; i < 6; ++i)
    if (counts[i] < 0) return FA_ERR_INVALID_ARG;
  if ((counts[1] > 0) != (counts[2] > 0) || (counts[4] > 0) != (counts[5] > 0))
    return FA_ERR_INVALID_ARG;
  const long long lines = (long long)B * H * ((N + fa::kMaskBlock - 1) / fa::kMaskBlock);
  if ((long long)B * H * N > 0 && (counts[0] < lines || counts[3] < lines || !plan || !aligned4(plan)))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}
}  // namespace

int fa_sparse_plan(const unsigned char* host_mask, long long mask_stride_b, long long mask_stride_h,
                   int B, int H, int N, int causal, int* plan, long long plan_ints, int* counts) {
  if (B < 0 || H < 0 || N < 0 || (causal != 0 && causal != 1) || !counts) return FA_ERR_INVALID_ARG;
  if (mask_stride_b < 0 || mask_stride_h < 0) return FA_ERR_INVALID_ARG;
  const int nb = (N + fa::kMaskBlock - 1) / fa::kMaskBlock;
  if (nb > fa::kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N > 0 && !host_mask) return FA_ERR_INVALID_ARG;
  std::vector<SparseItem> ci, ri;
  std::vector<int> cc, rc;
  int cs = 0, rs = 0;
  if (N > 0) {
    sparse_pieces(host_mask, mask_stride_b, mask_stride_h, B, H, nb, causal, true, ci, cc, &cs);
    sparse_pieces(host_mask, mask_stride_b, mask_stride_h, B, H, nb, causal, false, ri, rc, &rs);
  }
  const int c[8] = {(int)ci.size(), (int)cc.size() / 4, cs, (int)ri.size(), (int)rc.size() / 4, rs, 0, 0};
  std::copy(c, c + 8, counts);
  if (!plan) return FA_OK;  // counts only
  const long long need = 4LL * (c[0] + c[1] + c[3] + c[4]);
  if (plan_ints < need) return FA_ERR_INVALID_ARG;
  int* w = plan;
  for (const auto& it : ci) { *w++ = it.bh; *w++ = it.blk; *w++ = it.first; *w++ = it.slot; }
  w = std::copy(cc.begin(), cc.end(), w);
  for (const auto& it : ri) { *w++ = it.bh; *w++ = it.blk; *w++ = it.first; *w++ = it.slot; }
  std::copy(rc.begin(), rc.end(), w);
  return FA_OK;
}

size_t fa_fwd_sparse_planned_workspace_bytes(int B, int H, int N, int d, const int* counts) {
  if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128) || !counts || counts[5] < 0) return 0;
  return (size_t)counts[5] * fa::kMaskBlock * (size_t)(d + 1) * sizeof(float);
}

int fa_fwd_sparse_planned(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int H, int N, int d, float scale, int causal, const int* kv_len,
                          const unsigned char* block_mask, long long mask_stride_b,
                          long long mask_stride_h, const int* plan, const int* counts,
                          void* workspace, size_t workspace_bytes, void* stream, int in_dtype,
                          int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if ((N + fa::kMaskBlock - 1) / fa::kMaskBlock > fa::kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  if (mask_stride_b < 0 || mask_stride_h < 0) return FA_ERR_INVALID_ARG;
  if ((st = check_plan(B, H, N, plan, counts)) != FA_OK) return st;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse || !block_mask) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  if (counts[5] > 0 && (!workspace || !aligned16(workspace) ||
                        workspace_bytes < fa_fwd_sparse_planned_workspace_bytes(B, H, N, d, counts)))
    return FA_ERR_WORKSPACE;
  const int* row_items = plan + 4LL * (counts[0] + counts[1]);
  fa::FwdArgs a{q, k, v, o, lse, kv_len, B, H, N, d, scale, causal, N, 0, 0, 1, N, 0, 0, H,
                block_mask, mask_stride_b, mask_stride_h, row_items, row_items + 4LL * counts[3],
                counts[3], counts[4], counts[5], (float*)workspace};
  hipError_t e = fa::launch_fwd_mfma_sparse(a, elem(in_dtype), elem(o_dtype), (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_sparse_planned_workspace_bytes(int B, int H, int N, int d, const int* counts) {
  if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128) || !counts || counts[2] < 0 || counts[5] < 0)
    return 0;
  return dsum_bytes_aligned(B, H, N) +
         up256(2 * (size_t)counts[2] * fa::kMaskBlock * (size_t)d * sizeof(float)) +
         (size_t)counts[5] * fa::kMaskBlock * (size_t)d * sizeof(float);
}

int fa_bwd_sparse_planned(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                          int H, int N, int d, float scale, int causal, const int* kv_len,
                          const unsigned char* block_mask, long long mask_stride_b,
                          long long mask_stride_h, const int* plan, const int* counts,
                          void* workspace, size_t workspace_bytes, void* stream, int dtype,
                          int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!o_dtype_ok(dtype, o_dtype)) return FA_ERR_UNSUPPORTED;
  if ((N + fa::kMaskBlock - 1) / fa::kMaskBlock > fa::kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  if (mask_stride_b < 0 || mask_stride_h < 0) return FA_ERR_INVALID_ARG;
  if ((st = check_plan(B, H, N, plan, counts)) != FA_OK) return st;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !block_mask)
    return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < fa_bwd_sparse_planned_workspace_bytes(B, H, N, d, counts))
    return FA_ERR_WORKSPACE;
  char* w = (char*)workspace;
  float* kv_part = (float*)(w + dsum_bytes_aligned(B, H, N));
  float* q_part = (float*)((char*)kv_part + up256(2 * (size_t)counts[2] * fa::kMaskBlock * d * 4));
  const int* col_items = plan;
  const int* cols = plan + 4LL * counts[0];
  const int* row_items = cols + 4LL * counts[1];
  const int* rows = row_items + 4LL * counts[3];
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, kv_len, B, H, N, d, scale,
                causal, H, 1, kv_part, block_mask, mask_stride_b, mask_stride_h, col_items, cols,
                counts[0], counts[1], counts[2], row_items, rows, counts[3], counts[4], counts[5],
                q_part};
  a.o_f32 = o_dtype == FA_F32 ? 1 : 0;
  hipError_t e = fa::launch_bwd_mfma_sparse(a, elem(dtype),
                                            (int)fa::BwdStage::DQ | (int)fa::BwdStage::DKDV,
                                            (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fp8_quantize(const void* q, const void* k, const void* v, const signed char* signs,
                    unsigned char* q8, unsigned char* k8, unsigned char* vt8, float* q_scale,
                    float* k_scale, float* v_scale, float* v_amax, int B, int H, int N, int d,
                    void* stream, int in_dtype) {
  int st = check_scalars(B, H, N, d, 1.f, 0);
  if (st != FA_OK) return st;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !q8 || !k8 || !vt8 || !q_scale || !k_scale || !v_scale || !v_amax)
    return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(k8) ||
      !aligned16(vt8) || !aligned4(q_scale) || !aligned4(k_scale) || !aligned4(v_scale) ||
      !aligned4(v_amax))
    return FA_ERR_INVALID_ARG;
  fa::Fp8QuantArgs a{q, k, v, signs, q8, k8, vt8, q_scale, k_scale, v_scale, v_amax,
                     B, H, N, d, fp8_sizes(B, H, N, d).Np};
  hipError_t e = fa::launch_fp8_quantize(a, elem(in_dtype), (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const unsigned char* q8, const unsigned char* k8, const unsigned char* vt8,
               const float* q_scale, const float* k_scale, const float* v_scale, int rotated,
               void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
               const int* kv_len, void* stream, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!dtype_ok(o_dtype)) return FA_ERR_UNSUPPORTED;
  if (rotated != 0 && rotated != 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q8 || !k8 || !vt8 || !q_scale || !k_scale || !v_scale || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(vt8) || !aligned4(q_scale) ||
      !aligned4(k_scale) || !aligned4(v_scale) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  fa::Fp8FwdArgs a{q8, k8, vt8, q_scale, k_scale, v_scale, o, lse, kv_len, B, H, N, d,
                   fp8_sizes(B, H, N, d).Np, scale, causal, rotated, o_dtype == FA_BF16 ? 1 : 0};
  hipError_t e = fa::launch_fwd_fp8(a, elem(o_dtype), (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_fp8_workspace_bytes(int B, int H, int N, int d) {
  if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128)) return 0;
  const Fp8Sizes z = fp8_sizes(B, H, N, d);
  return 2 * up256(z.qk) + up256(z.vt) + up256(z.nq * 4) + up256(z.nk * 4) + up256(z.bh * 4) +
         up256(z.nk * 4);
}

int fa_fwd_fp8_incoherent(const void* q, const void* k, const void* v, const signed char* signs,
                          void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
                          const int* kv_len, void* workspace, size_t workspace_bytes, void* stream,
                          int in_dtype, int o_dtype) {
  int st = check_scalars(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (kv_len && !aligned4(kv_len)) return FA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < fa_fwd_fp8_workspace_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  const Fp8Sizes z = fp8_sizes(B, H, N, d);
  unsigned char* w = (unsigned char*)workspace;
  unsigned char* q8 = w;
  unsigned char* k8 = q8 + up256(z.qk);
  unsigned char* vt8 = k8 + up256(z.qk);
  float* qs = (float*)(vt8 + up256(z.vt));
  float* ks = (float*)((unsigned char*)qs + up256(z.nq * 4));
  float* vs = (float*)((unsigned char*)ks + up256(z.nk * 4));
  float* va = (float*)((unsigned char*)vs + up256(z.bh * 4));
  st = fa_fp8_quantize(q, k, v, signs, q8, k8, vt8, qs, ks, vs, va, B, H, N, d, stream, in_dtype);
  if (st != FA_OK) return st;
  return fa_fwd_fp8(q8, k8, vt8, qs, ks, vs, signs ? 1 : 0, o, lse, B, H, N, d, scale, causal,
                    kv_len, stream, o_dtype);
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success (work enqueued)";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: null or misaligned pointer, negative size, bad scale or flag";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim must be 64 or 128; dtype pair not supported";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing, misaligned or smaller than the entry point's *_workspace_bytes()";
    case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
    case FA_ERR_TOO_LARGE: return "FA_ERR_TOO_LARGE: B*H*N exceeds FA_NOALLOC_MAX_ROWS, the built-in scratch of fa_bwd_noalloc";
    default: return "unknown fa status";
  }
}

}  // extern "C"
