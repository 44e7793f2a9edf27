// Backward exact attention for bf16 / fp16 inputs on gfx950 MFMA.
//
// The forward keeps only O and one log-sum-exp per query row; the backward
// rebuilds each probability tile P = exp(scale * Q K^T - LSE) from Q, K and
// LSE instead of reading a stored N x N matrix (marketmaker.cc article
// "Flash attention and the sequence-length question", section
// "向后传递：重新计算而不是存储"; Ultralytics glossary page, section "Come
// funziona Flash Attention"; delect.ru glossary, section "Что подтверждено").
// The pages give no gradient formulas; these are the chain rule through
// O = P V and the row softmax:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three launches, no atomics, so the result is bit-reproducible:
//   1. dsum_kernel:  D_i = rowsum(dO * O) into the caller's workspace.
//   2. dkdv_kernel:  one workgroup per key block; K and V stay in VGPRs, the
//      loop streams query tiles (Q, dO, LSE, D) through LDS. Per tile:
//      S = Q K^T and dP = dO V^T with the key as the accumulator column (lane),
//      so P and dS come out of the accumulator already in the layout the
//      next two products take as B operand: dV^T += dO^T P, dK^T += Q^T dS.
//   3. dq_kernel: one workgroup per query block; Q and dO stay in VGPRs, the
//      loop streams key tiles (K, V) through LDS. Per tile: S^T = K Q^T and
//      dP^T = V dO^T with the query as the lane, then dQ^T += K^T dS^T.
// Kernel 3 recomputes S and dP, so the MFMA work is 7 products per tile pair
// against the 5 the gradients need.
#include "fa_internal.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic (fp32). LPR lanes share a row, 16 bytes each.
template <typename T, int D>
__global__ __launch_bounds__(256) void dsum_kernel(const uint16_t* __restrict__ o,
                                                   const uint16_t* __restrict__ dout,
                                                   float* __restrict__ dsum, long rows) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + tid / LPR;
  const int part = tid % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 ov = *(const u32x4*)(o + row * D + part * 8);
    const u32x4 gv = *(const u32x4*)(dout + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(Mfma<T>::to_f32(ov[i] & 0xffffu), Mfma<T>::to_f32(gv[i] & 0xffffu), acc);
      acc = fmaf(Mfma<T>::to_f32(ov[i] >> 16), Mfma<T>::to_f32(gv[i] >> 16), acc);
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) dsum[row] = acc;
}

// Load 4 consecutive rows x 8 columns (16 bytes per row) of a [N, D] tile.
template <int D>
__device__ inline void load_unit(const uint16_t* __restrict__ base, int row0, int c8, int valid,
                                 u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (row0 + i < valid) ? *(const u32x4*)(base + (size_t)(row0 + i) * D + c8 * 8)
                              : u32x4{0u, 0u, 0u, 0u};
  }
}

// Store a 4x8 unit row-major (stride RLD) at (row0, 8*c8).
__device__ inline void store_rows(uint16_t* dst, int RLD, int row0, int c8, const u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u32x4*)&dst[(row0 + i) * RLD + c8 * 8] = r[i];
}

// Store a 4x8 unit transposed: for each of the 8 columns, the 4 rows as one
// 8-byte run at [col][row0 .. row0+3] (stride TLD).
__device__ inline void store_cols(uint16_t* dst, int TLD, int row0, int c8, const u32x4 (&r)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t w0 = r[0][p], w1 = r[1][p], w2 = r[2][p], w3 = r[3][p];
    const u32x2 lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
    const u32x2 hi = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
    *(u32x2*)&dst[(c8 * 8 + 2 * p) * TLD + row0] = lo;
    *(u32x2*)&dst[(c8 * 8 + 2 * p + 1) * TLD + row0] = hi;
  }
}

// A fragment from a transposed tile: row `m` of the transpose, 16 reduction
// indices starting at k0, taken as runs [k0+4h, +4) and [k0+8+4h, +4) — the
// order in which a 32x32 accumulator holds them in lane half h.
__device__ inline u32x4 frag_cols(const uint16_t* src, int TLD, int m, int k0, int hh) {
  const uint16_t* p = &src[m * TLD + k0 + 4 * hh];
  const u32x2 a = *(const u32x2*)p;
  const u32x2 b = *(const u32x2*)(p + 8);
  return u32x4{a.x, a.y, b.x, b.y};
}

template <typename T>
__device__ inline u32x4 pack8(const f32x16& x, int base) {
  return u32x4{Mfma<T>::pack(x[base + 0], x[base + 1]), Mfma<T>::pack(x[base + 2], x[base + 3]),
               Mfma<T>::pack(x[base + 4], x[base + 5]), Mfma<T>::pack(x[base + 6], x[base + 7])};
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (b, h, key block of 32 * WA keys).
template <int D>
struct DkdvCfg {
  static constexpr int WA = (D == 128) ? 4 : 4;
  static constexpr int MINB = (D == 128) ? 1 : 2;
};

template <typename T, int D>
__global__ __launch_bounds__(64 * DkdvCfg<D>::WA, DkdvCfg<D>::MINB) void dkdv_kernel(BwdArgs a) {
  constexpr int WA = DkdvCfg<D>::WA;
  constexpr int NT = 64 * WA;
  constexpr int BK = 32 * WA;  // keys per workgroup
  constexpr int BQ = 32;       // queries per tile
  constexpr int DC = D / 16;
  constexpr int DT = D / 32;
  constexpr int RLD = D + 8;   // row-major tile stride (u16)
  constexpr int TLD = BQ + 4;  // transposed tile stride (u16)
  constexpr int UPT = (BQ / 4) * (D / 8);  // 4x8 units per tensor per tile
  static_assert(2 * UPT <= NT, "one unit per thread at most");

  __shared__ __attribute__((aligned(16))) uint16_t Qr[2][BQ * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t Gr[2][BQ * RLD];  // dO rows
  __shared__ __attribute__((aligned(16))) uint16_t Qt[2][D * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t Gt[2][D * TLD];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];  // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];  // D_i

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kl = lane & 31;
  const int hh = lane >> 5;

  const int N = a.N;
  const int nkb = (N + BK - 1) / BK;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nkb;
  const int kb = logical % nkb;  // causal: key block 0 has the most work, and runs first
  const int b = bh / a.H;

  const size_t head_off = (size_t)bh * N * D;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + head_off;
  const uint16_t* __restrict__ Kg = (const uint16_t*)a.k + head_off;
  const uint16_t* __restrict__ Vg = (const uint16_t*)a.v + head_off;
  const uint16_t* __restrict__ Gg = (const uint16_t*)a.dout + head_off;
  const float* __restrict__ Lg = a.lse + (size_t)bh * N;
  const float* __restrict__ Dg = a.dsum + (size_t)bh * N;

  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);

  const int key0 = kb * BK + wave * 32;
  const int my_key = key0 + kl;

  u32x4 kf[DC], vf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    const bool ok = my_key < kv_end;
    kf[dc] = ok ? *(const u32x4*)(Kg + (size_t)my_key * D + dc * 16 + hh * 8) : u32x4{0u, 0u, 0u, 0u};
    vf[dc] = ok ? *(const u32x4*)(Vg + (size_t)my_key * D + dc * 16 + hh * 8) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  // Query tiles this key block can contribute to.
  const int blk_key0 = kb * BK;
  const bool any_key = blk_key0 < kv_end;
  const int qt_begin = (a.causal ? blk_key0 : 0) / BQ;
  const int qt_end = any_key ? (N + BQ - 1) / BQ : qt_begin;
  const float sl2 = a.scale * kLog2e;

  // Prefetch registers: one 4x8 unit of Q or dO per thread, plus LSE/D.
  u32x4 ureg[4];
  float sreg = 0.f;
  const bool unit_thread = tid < 2 * UPT;
  const int ut = tid % UPT;
  const int ug = ut % (BQ / 4);
  const int uc8 = ut / (BQ / 4);
  const uint16_t* usrc = (tid < UPT) ? Qg : Gg;

  auto load_tile = [&](int it) {
    const int q0 = it * BQ;
    if (unit_thread) load_unit<D>(usrc, q0 + 4 * ug, uc8, N, ureg);
    if (tid < 2 * BQ) {
      const int q = q0 + (tid % BQ);
      float x = 0.f;
      if (q < N) x = (tid < BQ) ? Lg[q] * kLog2e : Dg[q];
      // rows without any visible key carry LSE = -inf; their P is masked to
      // zero, so a finite stand-in avoids inf - inf.
      sreg = (x == -INFINITY) ? 0.f : x;
    }
  };
  auto store_tile = [&](int buf) {
    if (unit_thread) {
      uint16_t* rdst = (tid < UPT) ? Qr[buf] : Gr[buf];
      uint16_t* tdst = (tid < UPT) ? Qt[buf] : Gt[buf];
      store_rows(rdst, RLD, 4 * ug, uc8, ureg);
      store_cols(tdst, TLD, 4 * ug, uc8, ureg);
    }
    if (tid < 2 * BQ) {
      if (tid < BQ) Ls[buf][tid] = sreg;
      else Ds[buf][tid - BQ] = sreg;
    }
  };

  if (qt_begin < qt_end) load_tile(qt_begin);
  for (int it = qt_begin; it < qt_end; ++it) {
    const int buf = (it - qt_begin) & 1;
    store_tile(buf);
    __syncthreads();
    if (it + 1 < qt_end) load_tile(it + 1);

    const int q0 = it * BQ;
    // Skip tiles wholly before this wave's first key (causal) or past its keys.
    const bool wave_live = (key0 < kv_end) && (!a.causal || q0 + BQ - 1 >= key0);
    if (wave_live) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4 qa = *(const u32x4*)&Qr[buf][kl * RLD + dc * 16 + hh * 8];
        s = Mfma<T>::mma32(qa, kf[dc], s);
      }
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4 ga = *(const u32x4*)&Gr[buf][kl * RLD + dc * 16 + hh * 8];
        dp = Mfma<T>::mma32(ga, vf[dc], dp);
      }
      const bool need_mask = (q0 + BQ > N) || (key0 + 32 > kv_end) || (a.causal && key0 + 31 > q0);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qi = 8 * r4 + 4 * hh;
        const f32x4 l4 = *(const f32x4*)&Ls[buf][qi];
        const f32x4 d4 = *(const f32x4*)&Ds[buf][qi];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          float p = fast_exp2(fmaf(s[r], sl2, -l4[e]));
          if (need_mask) {
            const int q = q0 + qi + e;
            const bool vis = (q < N) && (my_key < kv_end) && (!a.causal || my_key <= q);
            p = vis ? p : 0.f;
          }
          s[r] = p;
          dp[r] = p * (dp[r] - d4[e]);
        }
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 pf = pack8<T>(s, 8 * c2);
        const u32x4 sf = pack8<T>(dp, 8 * c2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4 ga = frag_cols(Gt[buf], TLD, dt * 32 + kl, 16 * c2, hh);
          dv[dt] = Mfma<T>::mma32(ga, pf, dv[dt]);
          const u32x4 qa = frag_cols(Qt[buf], TLD, dt * 32 + kl, 16 * c2, hh);
          dk[dt] = Mfma<T>::mma32(qa, sf, dk[dt]);
        }
      }
    }
  }

  // dK^T / dV^T accumulators: lane = key, registers = d in runs of 4.
  if (my_key < N) {
    uint16_t* dKg = (uint16_t*)a.dk + head_off + (size_t)my_key * D;
    uint16_t* dVg = (uint16_t*)a.dv + head_off + (size_t)my_key * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + r4 * 8 + 4 * hh;
        const f32x16& K4 = dk[dt];
        const f32x16& V4 = dv[dt];
        *(u32x2*)(dKg + d0) = u32x2{Mfma<T>::pack(K4[4 * r4] * a.scale, K4[4 * r4 + 1] * a.scale),
                                    Mfma<T>::pack(K4[4 * r4 + 2] * a.scale, K4[4 * r4 + 3] * a.scale)};
        *(u32x2*)(dVg + d0) = u32x2{Mfma<T>::pack(V4[4 * r4], V4[4 * r4 + 1]),
                                    Mfma<T>::pack(V4[4 * r4 + 2], V4[4 * r4 + 3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, h, query block of 128 rows).
template <int D>
struct DqCfg {
  static constexpr int BC = (D == 128) ? 32 : 64;  // keys per tile
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdArgs a) {
  constexpr int NT = 256;
  constexpr int BR = 128;
  constexpr int BC = DqCfg<D>::BC;
  constexpr int KT = BC / 32;
  constexpr int DC = D / 16;
  constexpr int DT = D / 32;
  constexpr int RLD = D + 8;
  constexpr int TLD = BC + 4;
  constexpr int UPT = (BC / 4) * (D / 8);
  static_assert(2 * UPT == NT, "one unit of K or V per thread");

  __shared__ __attribute__((aligned(16))) uint16_t Kr[2][BC * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vr[2][BC * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][D * TLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ql = lane & 31;
  const int hh = lane >> 5;

  const int N = a.N;
  const int nqb = (N + BR - 1) / BR;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqb;
  int qb = logical % nqb;
  if (a.causal) qb = nqb - 1 - qb;
  const int b = bh / a.H;

  const size_t head_off = (size_t)bh * N * D;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + head_off;
  const uint16_t* __restrict__ Kg = (const uint16_t*)a.k + head_off;
  const uint16_t* __restrict__ Vg = (const uint16_t*)a.v + head_off;
  const uint16_t* __restrict__ Gg = (const uint16_t*)a.dout + head_off;

  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  const int q_blk0 = qb * BR;
  int kv_lim = kv_end;
  if (a.causal) kv_lim = min(kv_lim, min(q_blk0 + BR, N));
  const int ntiles = (kv_lim + BC - 1) / BC;

  const int wq0 = q_blk0 + wave * 32;
  const int my_q = wq0 + ql;
  int w_lim = kv_end;
  if (a.causal) w_lim = min(w_lim, min(wq0 + 31, N - 1) + 1);

  u32x4 qf[DC], gf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    const bool ok = my_q < N;
    qf[dc] = ok ? *(const u32x4*)(Qg + (size_t)my_q * D + dc * 16 + hh * 8) : u32x4{0u, 0u, 0u, 0u};
    gf[dc] = ok ? *(const u32x4*)(Gg + (size_t)my_q * D + dc * 16 + hh * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  float lse2 = 0.f, dsum = 0.f;
  if (my_q < N) {
    const float l = a.lse[(size_t)bh * N + my_q];
    lse2 = (l == -INFINITY) ? 0.f : l * kLog2e;
    dsum = a.dsum[(size_t)bh * N + my_q];
  }
  const float sl2 = a.scale * kLog2e;

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};

  u32x4 ureg[4];
  const int ut = tid % UPT;
  const int ug = ut % (BC / 4);
  const int uc8 = ut / (BC / 4);
  const bool is_k = tid < UPT;
  const uint16_t* usrc = is_k ? Kg : Vg;

  auto load_tile = [&](int j) { load_unit<D>(usrc, j * BC + 4 * ug, uc8, kv_end, ureg); };
  auto store_tile = [&](int buf) {
    if (is_k) {
      store_rows(Kr[buf], RLD, 4 * ug, uc8, ureg);
      store_cols(Kt[buf], TLD, 4 * ug, uc8, ureg);
    } else {
      store_rows(Vr[buf], RLD, 4 * ug, uc8, ureg);
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
      f32x16 s[KT], dp[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = f32x16{};
        dp[kt] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const u32x4 ka = *(const u32x4*)&Kr[buf][(kt * 32 + ql) * RLD + dc * 16 + hh * 8];
          s[kt] = Mfma<T>::mma32(ka, qf[dc], s[kt]);
        }
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const u32x4 va = *(const u32x4*)&Vr[buf][(kt * 32 + ql) * RLD + dc * 16 + hh * 8];
          dp[kt] = Mfma<T>::mma32(va, gf[dc], dp[kt]);
        }
      }
      const bool need_mask = (t0 + BC > kv_end) || (my_q >= N) || (a.causal && t0 + BC - 1 > wq0);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(s[kt][r], sl2, -lse2));
          if (need_mask) {
            const int key = t0 + kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool vis = (my_q < N) && key < kv_end && (!a.causal || key <= my_q);
            p = vis ? p : 0.f;
          }
          dp[kt][r] = p * (dp[kt][r] - dsum);
        }
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const u32x4 sf = pack8<T>(dp[kt], 8 * c2);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const u32x4 ka = frag_cols(Kt[buf], TLD, dt * 32 + ql, kt * 32 + 16 * c2, hh);
            dq[dt] = Mfma<T>::mma32(ka, sf, dq[dt]);
          }
        }
      }
    }
  }

  if (my_q < N) {
    uint16_t* dQg = (uint16_t*)a.dq + head_off + (size_t)my_q * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + r4 * 8 + 4 * hh;
        const f32x16& Q4 = dq[dt];
        *(u32x2*)(dQg + d0) = u32x2{Mfma<T>::pack(Q4[4 * r4] * a.scale, Q4[4 * r4 + 1] * a.scale),
                                    Mfma<T>::pack(Q4[4 * r4 + 2] * a.scale, Q4[4 * r4 + 3] * a.scale)};
      }
    }
  }
}

template <typename T, int D>
hipError_t launch(const BwdArgs& a, int stages, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (stages & (int)BwdStage::DSUM) {
    const long rows = (long)a.B * a.H * a.N;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((dsum_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       st, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.dsum, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & (int)BwdStage::DKDV) {
    constexpr int WA = DkdvCfg<D>::WA;
    const long nkb = (a.N + 32 * WA - 1) / (32 * WA);
    hipLaunchKernelGGL((dkdv_kernel<T, D>), dim3((unsigned)((long)a.B * a.H * nkb)), dim3(64 * WA),
                       0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & (int)BwdStage::DQ) {
    const long nqb = (a.N + 127) / 128;
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3((unsigned)((long)a.B * a.H * nqb)), dim3(256), 0, st,
                       a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return e;
}

template <typename T>
hipError_t launch_t(const BwdArgs& a, int stages, hipStream_t st) {
  return (a.d == 128) ? launch<T, 128>(a, stages, st) : launch<T, 64>(a, stages, st);
}

}  // namespace

hipError_t launch_bwd_mfma(const BwdArgs& a, Elem t, int stages, hipStream_t st) {
  return (t == Elem::BF16) ? launch_t<BF16>(a, stages, st) : launch_t<F16>(a, stages, st);
}

}  // namespace fa
