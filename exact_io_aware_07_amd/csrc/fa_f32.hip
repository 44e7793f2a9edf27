// fp32 exact attention (forward and backward) on the gfx950 vector ALUs.
//
// Same tiled method as the MFMA kernels: K/V tiles staged through LDS, a
// running row max and row sum with the output rescaled whenever the max
// grows and divided by the row sum once at the end (marketmaker.cc article
// "Flash attention and the sequence-length question", sections "Flash
// 注意力算法" and "在线softmax递归"), and a backward that rebuilds P from Q, K
// and the stored LSE (section "向后传递：重新计算而不是存储"). Every product,
// exponential and sum is fp32; nothing is rounded to a narrower type.
//
// Work split: G = D / 32 lanes share one row (one query in the forward and
// dQ kernels, one key in the dK/dV kernel); each lane owns 32 of its d
// elements, and dot products are finished with G-lane shuffles.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kT = 256;
constexpr int kTile = 32;  // rows per LDS tile

template <int G>
__device__ inline float group_sum(float x) {
#pragma unroll
  for (int off = 1; off < G; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Partial row offset inside an LDS tile: lane part p reads columns
// [32p, 32p + 32) at p * 33 so the G parts fall in different banks.
template <int D>
struct F32Layout {
  static constexpr int G = D / 32;
  static constexpr int LD = G * 33;
};

template <int D>
__global__ __launch_bounds__(kT) void fwd_f32_kernel(FwdArgs a) {
  constexpr int G = F32Layout<D>::G;
  constexpr int LD = F32Layout<D>::LD;
  constexpr int QPB = kT / G;
  __shared__ float Ks[kTile * LD];
  __shared__ float Vs[kTile * LD];

  const int tid = threadIdx.x;
  const int part = tid % G;
  const int N = a.N;
  const int nqb = (N + QPB - 1) / QPB;
  const int bh = blockIdx.x / nqb;
  const int qb = blockIdx.x % nqb;
  const int b = bh / a.H;
  const size_t head_off = (size_t)bh * N * D;
  const float* Qg = (const float*)a.q + head_off;
  const float* Kg = (const float*)a.k + head_off;
  const float* Vg = (const float*)a.v + head_off;

  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  const int my_q = qb * QPB + tid / G;
  int kv_lim = kv_end;
  if (a.causal) kv_lim = min(kv_lim, min(qb * QPB + QPB, N));
  const int ntiles = (kv_lim + kTile - 1) / kTile;

  float q[32], o[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    q[e] = (my_q < N) ? Qg[(size_t)my_q * D + part * 32 + e] : 0.f;
    o[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;

  for (int j = 0; j < ntiles; ++j) {
    const int t0 = j * kTile;
    __syncthreads();
    for (int i = tid; i < kTile * D; i += kT) {
      const int r = i / D, c = i % D;
      const bool ok = t0 + r < kv_end;
      Ks[r * LD + (c / 32) * 33 + (c % 32)] = ok ? Kg[(size_t)(t0 + r) * D + c] : 0.f;
      Vs[r * LD + (c / 32) * 33 + (c % 32)] = ok ? Vg[(size_t)(t0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    float s[kTile];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kTile; ++jj) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc = fmaf(q[e], Ks[jj * LD + part * 33 + e], acc);
      acc = group_sum<G>(acc);
      const int key = t0 + jj;
      const bool vis = key < kv_end && (!a.causal || key <= my_q);
      s[jj] = vis ? acc : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == m_run) ? 1.f : fast_exp2((m_run - m_new) * sl2);
    const float mref = (m_new == -INFINITY) ? 0.f : m_new * sl2;
    float lsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < kTile; ++jj) {
      s[jj] = fast_exp2(fmaf(s[jj], sl2, -mref));
      lsum += s[jj];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      float acc = o[e] * alpha;
#pragma unroll
      for (int jj = 0; jj < kTile; ++jj) acc = fmaf(s[jj], Vs[jj * LD + part * 33 + e], acc);
      o[e] = acc;
    }
  }

  if (my_q < N) {
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    float* Og = (float*)a.o + head_off + (size_t)my_q * D + part * 32;
#pragma unroll
    for (int e = 0; e < 32; e += 4) *(f32x4*)(Og + e) = f32x4{o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
    if (part == 0)
      a.lse[(size_t)bh * N + my_q] = (l_run > 0.f) ? m_run * a.scale + logf(l_run) : -INFINITY;
  }
}

// D_i = rowsum(dO * O) in fp32.
template <int D>
__global__ __launch_bounds__(kT) void dsum_f32_kernel(const float* __restrict__ o,
                                                       const float* __restrict__ dout,
                                                       float* __restrict__ dsum, long rows) {
  constexpr int LPR = D / 4;
  constexpr int RPB = kT / LPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const f32x4 x = *(const f32x4*)(o + row * D + 4 * part);
    const f32x4 g = *(const f32x4*)(dout + row * D + 4 * part);
    acc = x[0] * g[0] + x[1] * g[1] + x[2] * g[2] + x[3] * g[3];
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) dsum[row] = acc;
}

// dK, dV: G lanes per key; query tiles stream through LDS.
template <int D>
__global__ __launch_bounds__(kT) void dkdv_f32_kernel(BwdArgs a) {
  constexpr int G = F32Layout<D>::G;
  constexpr int LD = F32Layout<D>::LD;
  constexpr int KPB = kT / G;
  __shared__ float Qs[kTile * LD];
  __shared__ float Gs[kTile * LD];
  __shared__ float Ls[kTile];
  __shared__ float Ds[kTile];

  const int tid = threadIdx.x;
  const int part = tid % G;
  const int N = a.N;
  const int nkb = (N + KPB - 1) / KPB;
  const int bh = blockIdx.x / nkb;
  const int kb = blockIdx.x % nkb;
  const int b = bh / a.H;
  const size_t head_off = (size_t)bh * N * D;
  const float* Qg = (const float*)a.q + head_off;
  const float* Kg = (const float*)a.k + head_off;
  const float* Vg = (const float*)a.v + head_off;
  const float* Gg = (const float*)a.dout + head_off;
  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  const int my_k = kb * KPB + tid / G;
  const bool key_ok = my_k < kv_end;

  float k[32], v[32], dk[32], dv[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    k[e] = key_ok ? Kg[(size_t)my_k * D + part * 32 + e] : 0.f;
    v[e] = key_ok ? Vg[(size_t)my_k * D + part * 32 + e] : 0.f;
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const float sl2 = a.scale * kLog2e;
  const int blk_k0 = kb * KPB;
  const int q_begin = (a.causal ? blk_k0 : 0) / kTile;
  const int q_end = (blk_k0 < kv_end) ? (N + kTile - 1) / kTile : q_begin;

  for (int it = q_begin; it < q_end; ++it) {
    const int q0 = it * kTile;
    __syncthreads();
    for (int i = tid; i < kTile * D; i += kT) {
      const int r = i / D, c = i % D;
      const bool ok = q0 + r < N;
      Qs[r * LD + (c / 32) * 33 + (c % 32)] = ok ? Qg[(size_t)(q0 + r) * D + c] : 0.f;
      Gs[r * LD + (c / 32) * 33 + (c % 32)] = ok ? Gg[(size_t)(q0 + r) * D + c] : 0.f;
    }
    if (tid < kTile) {
      const int q = q0 + tid;
      const float l = (q < N) ? a.lse[(size_t)bh * N + q] : 0.f;
      Ls[tid] = (l == -INFINITY) ? 0.f : l * kLog2e;
      Ds[tid] = (q < N) ? a.dsum[(size_t)bh * N + q] : 0.f;
    }
    __syncthreads();
    for (int ii = 0; ii < kTile; ++ii) {
      const int q = q0 + ii;
      float sdot = 0.f, gdot = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        sdot = fmaf(k[e], Qs[ii * LD + part * 33 + e], sdot);
        gdot = fmaf(v[e], Gs[ii * LD + part * 33 + e], gdot);
      }
      sdot = group_sum<G>(sdot);
      gdot = group_sum<G>(gdot);
      const bool vis = (q < N) && key_ok && (!a.causal || my_k <= q);
      const float p = vis ? fast_exp2(fmaf(sdot, sl2, -Ls[ii])) : 0.f;
      const float ds = p * (gdot - Ds[ii]);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        dv[e] = fmaf(p, Gs[ii * LD + part * 33 + e], dv[e]);
        dk[e] = fmaf(ds, Qs[ii * LD + part * 33 + e], dk[e]);
      }
    }
  }
  if (my_k < N) {
    float* dKg = (float*)a.dk + head_off + (size_t)my_k * D + part * 32;
    float* dVg = (float*)a.dv + head_off + (size_t)my_k * D + part * 32;
#pragma unroll
    for (int e = 0; e < 32; e += 4) {
      *(f32x4*)(dKg + e) = f32x4{dk[e] * a.scale, dk[e + 1] * a.scale, dk[e + 2] * a.scale, dk[e + 3] * a.scale};
      *(f32x4*)(dVg + e) = f32x4{dv[e], dv[e + 1], dv[e + 2], dv[e + 3]};
    }
  }
}

// dQ: G lanes per query; key tiles stream through LDS.
template <int D>
__global__ __launch_bounds__(kT) void dq_f32_kernel(BwdArgs a) {
  constexpr int G = F32Layout<D>::G;
  constexpr int LD = F32Layout<D>::LD;
  constexpr int QPB = kT / G;
  __shared__ float Ks[kTile * LD];
  __shared__ float Vs[kTile * LD];

  const int tid = threadIdx.x;
  const int part = tid % G;
  const int N = a.N;
  const int nqb = (N + QPB - 1) / QPB;
  const int bh = blockIdx.x / nqb;
  const int qb = blockIdx.x % nqb;
  const int b = bh / a.H;
  const size_t head_off = (size_t)bh * N * D;
  const float* Qg = (const float*)a.q + head_off;
  const float* Kg = (const float*)a.k + head_off;
  const float* Vg = (const float*)a.v + head_off;
  const float* Gg = (const float*)a.dout + head_off;
  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  const int my_q = qb * QPB + tid / G;
  int kv_lim = kv_end;
  if (a.causal) kv_lim = min(kv_lim, min(qb * QPB + QPB, N));
  const int ntiles = (kv_lim + kTile - 1) / kTile;

  float q[32], g[32], dq[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    q[e] = (my_q < N) ? Qg[(size_t)my_q * D + part * 32 + e] : 0.f;
    g[e] = (my_q < N) ? Gg[(size_t)my_q * D + part * 32 + e] : 0.f;
    dq[e] = 0.f;
  }
  // D_i = sum_c dO_ic O_ic for this row (G lanes share it), written to the
  // workspace for the dK/dV kernel, which runs after this one.
  float dsum = 0.f;
  if (my_q < N) {
    const float* Og = (const float*)a.o + head_off + (size_t)my_q * D + part * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) dsum = fmaf(Og[e], g[e], dsum);
  }
  dsum = group_sum<G>(dsum);
  float lse2 = 0.f;
  if (my_q < N) {
    const float l = a.lse[(size_t)bh * N + my_q];
    lse2 = (l == -INFINITY) ? 0.f : l * kLog2e;
    if (part == 0) a.dsum[(size_t)bh * N + my_q] = dsum;
  }
  const float sl2 = a.scale * kLog2e;

  for (int j = 0; j < ntiles; ++j) {
    const int t0 = j * kTile;
    __syncthreads();
    for (int i = tid; i < kTile * D; i += kT) {
      const int r = i / D, c = i % D;
      const bool ok = t0 + r < kv_end;
      Ks[r * LD + (c / 32) * 33 + (c % 32)] = ok ? Kg[(size_t)(t0 + r) * D + c] : 0.f;
      Vs[r * LD + (c / 32) * 33 + (c % 32)] = ok ? Vg[(size_t)(t0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < kTile; ++jj) {
      const int key = t0 + jj;
      float sdot = 0.f, gdot = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        sdot = fmaf(q[e], Ks[jj * LD + part * 33 + e], sdot);
        gdot = fmaf(g[e], Vs[jj * LD + part * 33 + e], gdot);
      }
      sdot = group_sum<G>(sdot);
      gdot = group_sum<G>(gdot);
      const bool vis = (my_q < N) && key < kv_end && (!a.causal || key <= my_q);
      const float p = vis ? fast_exp2(fmaf(sdot, sl2, -lse2)) : 0.f;
      const float ds = p * (gdot - dsum);
#pragma unroll
      for (int e = 0; e < 32; ++e) dq[e] = fmaf(ds, Ks[jj * LD + part * 33 + e], dq[e]);
    }
  }
  if (my_q < N) {
    float* dQg = (float*)a.dq + head_off + (size_t)my_q * D + part * 32;
#pragma unroll
    for (int e = 0; e < 32; e += 4)
      *(f32x4*)(dQg + e) = f32x4{dq[e] * a.scale, dq[e + 1] * a.scale, dq[e + 2] * a.scale, dq[e + 3] * a.scale};
  }
}

template <int D>
hipError_t fwd_launch(const FwdArgs& a, hipStream_t s) {
  constexpr int QPB = kT / (D / 32);
  const long nqb = (a.N + QPB - 1) / QPB;
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)((long)a.B * a.H * nqb)), dim3(kT), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_launch(const BwdArgs& a, int stages, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (stages & (int)BwdStage::DSUM) {
    const long rows = (long)a.B * a.H * a.N;
    constexpr int RPB = kT / (D / 4);
    hipLaunchKernelGGL(dsum_f32_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kT), 0, s,
                       (const float*)a.o, (const float*)a.dout, a.dsum, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  constexpr int PB = kT / (D / 32);
  const long nb = (a.N + PB - 1) / PB;
  if (stages & (int)BwdStage::DQ) {
    hipLaunchKernelGGL(dq_f32_kernel<D>, dim3((unsigned)((long)a.B * a.H * nb)), dim3(kT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & (int)BwdStage::DKDV) {
    hipLaunchKernelGGL(dkdv_f32_kernel<D>, dim3((unsigned)((long)a.B * a.H * nb)), dim3(kT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return e;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  return (a.d == 128) ? fwd_launch<128>(a, s) : fwd_launch<64>(a, s);
}

hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s) {
  return (a.d == 128) ? bwd_launch<128>(a, stages, s) : bwd_launch<64>(a, stages, s);
}

}  // namespace fa
