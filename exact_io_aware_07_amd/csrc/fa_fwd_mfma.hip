// Forward exact attention for bf16 / fp16 inputs on gfx950 MFMA.
//
// The method: split Q into row blocks and K, V into column blocks; for each
// query block stream every key/value block through on-chip memory, keep a
// running row max m and row sum l, rescale the partial output by
// exp(m_old - m_new) whenever the max grows, and divide by l once at the end
// (marketmaker.cc article "Flash attention and the sequence-length
// question", sections "Flash 注意力算法" and "在线softmax递归"; the division
// deferred to the end of the loop is the first FA2 change listed in its
// section "FA2：并行性", and the same deferred form appears in the Ultralytics
// glossary page's streaming example, section "Come funziona Flash Attention").
// The grid covers batch x head x query block (the second FA2 change: query
// blocks are parallel, which keeps the GPU busy at batch 1-4) and each wave
// owns its own query rows (the third FA2 change: no cross-wave reduction).
//
// gfx950 mapping
//  * workgroup = 4 waves = 128 query rows; wave w owns rows [32w, 32w+32).
//  * S^T = K Q^T on v_mfma_f32_32x32x16 (A = K tile from LDS, B = the wave's
//    Q rows held in VGPRs for the whole kernel). In the 32x32 accumulator
//    layout lane l holds query column l % 32 and 16 keys, so a query's row
//    max and row sum are in-lane plus one exchange with lane l ^ 32.
//  * O^T += V^T P^T on the same MFMA. The probabilities leave the S
//    accumulator already in B-operand order (lane l % 32 = query, keys in
//    runs of 4), so P never goes through LDS. V is written to LDS transposed,
//    in runs of 4 keys per d, so each A fragment is two 8-byte LDS reads.
//  * K/V tiles are double-buffered in LDS with one barrier per tile; the next
//    tile's global loads are in flight while the current tile is computed.
//  * Scores stay in raw units; exp2 of (s * scale * log2 e - m * scale *
//    log2 e) is one FMA and one v_exp_f32 per score.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;  // query rows per workgroup

template <int D>
struct FwdTile;
template <>
struct FwdTile<128> {
  static constexpr int BC = 64;  // keys per tile: K and V tiles are 16 KiB each
};
template <>
struct FwdTile<64> {
  static constexpr int BC = 128;
};

template <typename T, int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_kernel(FwdArgs a) {
  constexpr int BC = FwdTile<D>::BC;
  constexpr int KT = BC / 32;                        // 32-key sub-tiles
  constexpr int DC = D / 16;                         // 16-wide d chunks (S reduction)
  constexpr int DT = D / 32;                         // 32-wide d tiles of O^T
  constexpr int K_LD = D + 8;                        // u16 per K row in LDS (16 B pad)
  constexpr int VT_LD = BC + 4;                      // u16 per V^T row in LDS (8 B pad)
  constexpr int KCH = BC * D / 8 / kThreads;         // 16-byte K chunks per thread
  constexpr int VU = (BC / 4) * (D / 8) / kThreads;  // 4-row x 8-col V units per thread
  static_assert(KCH >= 1 && VU >= 1, "tile too small for the workgroup");
  static_assert(BC * D / 8 % kThreads == 0 && (BC / 4) * (D / 8) % kThreads == 0, "");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * K_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VT_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ql = lane & 31;  // query column within the wave
  const int hh = lane >> 5;  // k-group half of the wave

  const int N = a.N;
  const int nqb = (N + kBR - 1) / kBR;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqb;
  int qb = logical % nqb;
  if (a.causal) qb = nqb - 1 - qb;  // longest causal blocks first
  const int b = bh / a.H;

  const size_t head_off = (size_t)bh * N * D;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + head_off;
  const uint16_t* __restrict__ Kg = (const uint16_t*)a.k + head_off;
  const uint16_t* __restrict__ Vg = (const uint16_t*)a.v + head_off;

  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  const int q_blk0 = qb * kBR;
  const int q_blk_last = min(q_blk0 + kBR, N) - 1;
  int kv_lim = kv_end;  // keys the workgroup needs (exclusive)
  if (a.causal) kv_lim = min(kv_lim, q_blk_last + 1);
  const int ntiles = (kv_lim + BC - 1) / BC;

  const int wq0 = q_blk0 + wave * 32;
  const int my_q = wq0 + ql;
  int w_lim = kv_end;  // keys this wave needs (exclusive)
  if (a.causal) w_lim = min(w_lim, min(wq0 + 31, N - 1) + 1);

  u32x4 qf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    qf[dc] = (my_q < N) ? *(const u32x4*)(Qg + (size_t)my_q * D + dc * 16 + hh * 8)
                        : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;  // running max of raw scores (both halves agree)
  float l_run = 0.f;        // running sum over this half's keys
  const float sl2 = a.scale * kLog2e;

  u32x4 kreg[KCH];
  u32x4 vreg[VU][4];

  auto load_tile = [&](int j) {
    const int t0 = j * BC;
    const int rows = kv_end - t0;  // rows at or past kv_end load as zeros
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / (D / 8), c8 = c % (D / 8);
      kreg[i] = (r < rows) ? *(const u32x4*)(Kg + (size_t)(t0 + r) * D + c8 * 8)
                           : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + kThreads * i;
      const int g = u % (BC / 4), c8 = u / (BC / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        vreg[i][r] = (row < rows) ? *(const u32x4*)(Vg + (size_t)(t0 + row) * D + c8 * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / (D / 8), c8 = c % (D / 8);
      *(u32x4*)&Ks[buf][r * K_LD + c8 * 8] = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + kThreads * i;
      const int g = u % (BC / 4), c8 = u / (BC / 4);
#pragma unroll
      for (int p = 0; p < 4; ++p) {  // dword p holds columns 2p (low half) and 2p+1
        const uint32_t w0 = vreg[i][0][p], w1 = vreg[i][1][p];
        const uint32_t w2 = vreg[i][2][p], w3 = vreg[i][3][p];
        const u32x2 lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
        const u32x2 hi = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
        *(u32x2*)&Vt[buf][(c8 * 8 + 2 * p) * VT_LD + 4 * g] = lo;
        *(u32x2*)&Vt[buf][(c8 * 8 + 2 * p + 1) * VT_LD + 4 * g] = hi;
      }
    }
  };

  if (ntiles > 0) load_tile(0);

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    store_tile(buf);
    __syncthreads();
    if (j + 1 < ntiles) load_tile(j + 1);

    const int t0 = j * BC;
    if (t0 < w_lim) {
      // S^T tile: 32 keys x 32 queries per sub-tile, raw dot products.
      f32x16 s[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const u32x4 kf = *(const u32x4*)&Ks[buf][(kt * 32 + ql) * K_LD + dc * 16 + hh * 8];
          s[kt] = Mfma<T>::mma32(kf, qf[dc], s[kt]);
        }
      }

      const bool need_mask = (t0 + BC > kv_end) || (a.causal && t0 + BC - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t0 + kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool vis = key < kv_end && (!a.causal || key <= my_q);
            if (!vis) s[kt][r] = -INFINITY;
          }
        }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
      }
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == m_run) ? 1.f : fast_exp2((m_run - m_new) * sl2);
      const float mref = (m_new == -INFINITY) ? 0.f : m_new * sl2;
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kt][r], sl2, -mref));
          s[kt][r] = p;
          lsum += p;
        }
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      }

      // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const u32x4 pf = {Mfma<T>::pack(s[kt][8 * c2 + 0], s[kt][8 * c2 + 1]),
                            Mfma<T>::pack(s[kt][8 * c2 + 2], s[kt][8 * c2 + 3]),
                            Mfma<T>::pack(s[kt][8 * c2 + 4], s[kt][8 * c2 + 5]),
                            Mfma<T>::pack(s[kt][8 * c2 + 6], s[kt][8 * c2 + 7])};
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint16_t* vp = &Vt[buf][(dt * 32 + ql) * VT_LD + kt * 32 + c2 * 16 + 4 * hh];
            const u32x2 v0 = *(const u32x2*)vp;
            const u32x2 v1 = *(const u32x2*)(vp + 8);
            const u32x4 vf = {v0.x, v0.y, v1.x, v1.y};
            oacc[dt] = Mfma<T>::mma32(vf, pf, oacc[dt]);
          }
        }
      }
    }
  }

  const float l_tot = l_run + swap_halves(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (my_q < N) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + r4 * 8 + 4 * hh;
        const float o0 = oacc[dt][4 * r4 + 0] * inv, o1 = oacc[dt][4 * r4 + 1] * inv;
        const float o2 = oacc[dt][4 * r4 + 2] * inv, o3 = oacc[dt][4 * r4 + 3] * inv;
        if constexpr (OUT_F32) {
          float* Og = (float*)a.o + head_off;
          *(f32x4*)(Og + (size_t)my_q * D + d0) = f32x4{o0, o1, o2, o3};
        } else {
          uint16_t* Og = (uint16_t*)a.o + head_off;
          *(u32x2*)(Og + (size_t)my_q * D + d0) = u32x2{Mfma<T>::pack(o0, o1), Mfma<T>::pack(o2, o3)};
        }
      }
    }
    if (hh == 0) {
      a.lse[(size_t)bh * N + my_q] =
          (l_tot > 0.f) ? m_run * a.scale + fast_log2(l_tot) * kLn2 : -INFINITY;
    }
  }
}

template <typename T, int D, bool OF>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const long nqb = (a.N + kBR - 1) / kBR;
  const long total = (long)a.B * a.H * nqb;
  hipLaunchKernelGGL((fwd_mfma_kernel<T, D, OF>), dim3((unsigned)total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, bool of, hipStream_t s) {
  if (a.d == 128) return of ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
  return of ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a, Elem in, Elem out, hipStream_t s) {
  const bool of = (out == Elem::F32);
  if (in == Elem::BF16) return launch_t<BF16>(a, of, s);
  return launch_t<F16>(a, of, s);
}

}  // namespace fa
