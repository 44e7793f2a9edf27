// FP8 forward with incoherent processing on gfx950 (marketmaker.cc article,
// section "FA3：料斗力学", item 3: the vectors are rotated at random before a
// block-wise quantisation, which spreads outliers over the coordinates).
//
// Two steps, each its own launch pair:
//  1. Quantisation (HBM-bound). Every row of Q and K is multiplied by a +-1
//     sign vector and put through the unnormalised Walsh-Hadamard transform
//     in fp32 (stage h = 1, 2, ..., d/2: elements i and i + h with bit h of i
//     clear become a + b and a - b), then quantised to OCP e4m3 with one
//     fp32 scale per block (128 query rows, 64 key rows): scale = amax / 448,
//     code = rne(clamp(x * (448 / amax), +-448)). V is not rotated; it has
//     one scale per head and is stored transposed, [d][N rounded up to 64],
//     so the P V product reads keys contiguously.
//  2. Attention on the codes: S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_f32_32x32x64_f8f6f4 (64 fp8 products per lane per instruction),
//     online softmax in fp32 as in the bf16 forward, and P quantised to e4m3
//     as 256 p (the largest p is 1, so 256 p stays below 448 and keeps small
//     values normal). The unnormalised rotation makes Q'K'^T = d Q K^T, so
//     the scores carry an extra 1/d.
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kQThreads = 256;
constexpr float kE4m3Max = 448.f;

// Four fp32 values to four e4m3 bytes, a in the lowest (round to nearest
// even; the callers keep |x| <= 448, past which the conversion gives NaN).
__device__ inline unsigned pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ inline float clamp448(float x) { return fminf(fmaxf(x, -kE4m3Max), kE4m3Max); }

// Largest value over the workgroup (kQThreads threads), in every thread.
__device__ inline float block_max(float m, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kQThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// Rotation of the EPT = D / TPR elements of one row a thread holds (TPR
// consecutive threads share a row): stages with h < EPT inside the thread,
// the others with the thread whose part index differs in bit h / EPT (the
// thread with that bit set holds the b of each pair).
template <int D, int TPR>
__device__ inline void fwht_rows(float (&x)[D / TPR], int part) {
  constexpr int EPT = D / TPR;
#pragma unroll
  for (int h = 1; h < EPT; h *= 2) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int h = EPT; h < D; h *= 2) {
    const int pm = h / EPT;
    const bool upper = (part & pm) != 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const float o = __shfl_xor(x[i], pm);
      x[i] = upper ? (o - x[i]) : (x[i] + o);
    }
  }
}

// Loads EPT consecutive 16-bit elements (a multiple of 8) of row `row`
// starting at column c0, as fp32; rows past N read as zero.
template <typename T, int EPT>
__device__ inline void load_row(const uint16_t* base, int N, int D, int row, int c0, float (&x)[EPT]) {
  if (row < N) {
    const u32x4* p = (const u32x4*)(base + (size_t)row * D + c0);
#pragma unroll
    for (int i = 0; i < EPT / 8; ++i) {
      const u32x4 w = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = Mfma<T>::to_f32(w[j] & 0xffffu);
        x[8 * i + 2 * j + 1] = Mfma<T>::to_f32(w[j] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) x[i] = 0.f;
  }
}

// Step 1a: rotate and quantise a block of RB rows of Q or K (RB = 128 or
// 64), or (AMAX_ONLY) only take the largest |v| of a block of V rows.
template <typename T, int D, int RB, bool AMAX_ONLY>
__device__ inline void quant_block(const Fp8QuantArgs& a, const uint16_t* src, unsigned char* dst,
                                   float* scale_out, int bh, int ib, float* red) {
  constexpr int TPR = kQThreads / RB;
  constexpr int EPT = D / TPR;
  const int t = threadIdx.x;
  const int r = t / TPR, part = t % TPR;
  const int row = ib * RB + r;
  const uint16_t* head = src + (size_t)bh * a.N * D;
  float x[EPT];
  load_row<T, EPT>(head, a.N, D, row, part * EPT, x);
  // No signs: no rotation at all (plain block-wise quantisation).
  if constexpr (!AMAX_ONLY) {
    if (a.signs) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) x[i] *= (float)a.signs[part * EPT + i];
      fwht_rows<D, TPR>(x, part);
    }
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmaxf(m, fabsf(x[i]));
  const float amax = block_max(m, red);
  if constexpr (AMAX_ONLY) {
    if (t == 0) scale_out[ib] = amax;
    return;
  } else {
    const float inv = amax > 0.f ? __fdiv_rn(kE4m3Max, amax) : 0.f;
    if (t == 0) scale_out[ib] = amax > 0.f ? __fdiv_rn(amax, kE4m3Max) : 0.f;
    if (row < a.N) {
      u32x4* out = (u32x4*)(dst + ((size_t)bh * a.N + row) * D + part * EPT);
#pragma unroll
      for (int i = 0; i < EPT / 16; ++i) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 16 * i + 4 * j;
          w[j] = pack4(clamp448(x[e] * inv), clamp448(x[e + 1] * inv), clamp448(x[e + 2] * inv),
                       clamp448(x[e + 3] * inv));
        }
        out[i] = w;
      }
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kQThreads) void fp8_qk_kernel(Fp8QuantArgs a) {
  __shared__ float red[kQThreads / 64];
  const int BH = a.B * a.H;
  const int nq = (a.N + 127) / 128, nk = (a.N + 63) / 64;
  int bid = blockIdx.x;
  if (bid < BH * nq) {
    const int bh = bid / nq;
    quant_block<T, D, 128, false>(a, (const uint16_t*)a.q, a.q8, a.q_scale + (size_t)bh * nq, bh,
                                  bid - bh * nq, red);
    return;
  }
  bid -= BH * nq;
  if (bid < BH * nk) {
    const int bh = bid / nk;
    quant_block<T, D, 64, false>(a, (const uint16_t*)a.k, a.k8, a.k_scale + (size_t)bh * nk, bh,
                                 bid - bh * nk, red);
    return;
  }
  bid -= BH * nk;
  const int bh = bid / nk;
  quant_block<T, D, 64, true>(a, (const uint16_t*)a.v, nullptr, a.v_amax + (size_t)bh * nk, bh,
                              bid - bh * nk, red);
}

// Step 1b: V of one 64-key block with its head's scale, written transposed:
// vt8[bh][m][key] for the block's 64 keys (zero codes past N).
template <typename T, int D>
__global__ __launch_bounds__(kQThreads) void fp8_v_kernel(Fp8QuantArgs a) {
  __shared__ float red[kQThreads / 64];
  __shared__ unsigned char tile[64][D + 4];
  const int nk = (a.N + 63) / 64;
  const int bh = blockIdx.x / nk, ib = blockIdx.x - bh * nk;
  const int t = threadIdx.x;
  float m = 0.f;
  for (int i = t; i < nk; i += kQThreads) m = fmaxf(m, a.v_amax[(size_t)bh * nk + i]);
  const float amax = block_max(m, red);
  const float inv = amax > 0.f ? __fdiv_rn(kE4m3Max, amax) : 0.f;
  if (ib == 0 && t == 0) a.v_scale[bh] = amax > 0.f ? __fdiv_rn(amax, kE4m3Max) : 0.f;
  constexpr int EPT = D / 4;
  const int r = t / 4, part = t % 4;
  float x[EPT];
  load_row<T, EPT>((const uint16_t*)a.v + (size_t)bh * a.N * D, a.N, D, ib * 64 + r, part * EPT, x);
#pragma unroll
  for (int i = 0; i < EPT / 4; ++i) {
    const unsigned w = pack4(clamp448(x[4 * i] * inv), clamp448(x[4 * i + 1] * inv),
                             clamp448(x[4 * i + 2] * inv), clamp448(x[4 * i + 3] * inv));
    *(unsigned*)&tile[r][part * EPT + 4 * i] = w;
  }
  __syncthreads();
  // D rows of 64 key bytes; each thread writes 64 * D / 256 = D / 4 bytes.
  constexpr int BPT = D / 4;               // bytes per thread (16 or 32)
  constexpr int TPM = 64 / BPT;            // threads per row of V^T
  const int mrow = t / TPM, k0 = (t % TPM) * BPT;
  unsigned char* out = a.vt8 + ((size_t)bh * D + mrow) * a.Np + (size_t)ib * 64 + k0;
#pragma unroll
  for (int i = 0; i < BPT / 16; ++i) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = k0 + 16 * i + 4 * j;
      w[j] = (unsigned)tile[kk][mrow] | ((unsigned)tile[kk + 1][mrow] << 8) |
             ((unsigned)tile[kk + 2][mrow] << 16) | ((unsigned)tile[kk + 3][mrow] << 24);
    }
    *(u32x4*)(out + 16 * i) = w;
  }
}

// ---------------------------------------------------------------------------
// Step 2: attention on the codes. One workgroup per (b, h, 128-query block),
// four waves of 32 queries; 64-key tiles of K (rows) and V^T (64-byte rows of
// keys) go HBM -> LDS directly, double-buffered, the next tile's copies in
// flight while the current one is computed.
//
// LDS tiles are rows of R bytes (R = D for K, 64 for V^T) in 16-byte chunks;
// logical chunk c of row r sits at position c ^ ((r / (256 / R)) % (R / 16)).
// A 16-byte read is served 16 lanes at a time; 16 lanes reading one chunk of
// 16 consecutive rows then cover the 16 chunk positions of a 256-byte bank
// window exactly once.
template <int R>
struct Fp8Tile {
  static constexpr int CPR = R / 16;
  static constexpr int RPW = 256 / R;  // rows per 256-byte bank window
  __device__ static int off(int row, int chunk) {
    return row * R + ((chunk ^ ((row / RPW) % CPR)) << 4);
  }
};

// One wave's share of a 64 x D-byte tile: lane i of wave instruction g fills
// bytes [1024 G + 16 i, +16) of the tile (G = wave * per_wave + g); that
// position holds logical chunk (i % CPR) ^ swizzle of row (1024 G + 16 i) / R.
template <int R, int ROWS>
__device__ inline void load_fp8_tile(__amdgpu_buffer_rsrc_t rs, unsigned char* dst, size_t row_stride,
                                     size_t col0, int wave, int lane) {
  constexpr int INSTR = ROWS * R / 1024;
  constexpr int PER_WAVE = INSTR / 4;
  static_assert(PER_WAVE >= 1 && INSTR % 4 == 0, "tile too small for four waves");
#pragma unroll
  for (int g = 0; g < PER_WAVE; ++g) {
    const int G = wave * PER_WAVE + g;
    const int pos = G * 1024 + 16 * lane;
    const int row = pos / R;
    const int chunk = ((pos % R) / 16) ^ ((row / Fp8Tile<R>::RPW) % Fp8Tile<R>::CPR);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(dst + G * 1024), 16,
        (int)(row * row_stride + col0 + 16 * chunk), 0, 0, 0);
  }
}

template <int D>
struct Fp8Cfg {
  static constexpr int OCC = 2;  // workgroups per CU the kernel is built for
};

__device__ inline i32x8 read32(const unsigned char* p0, const unsigned char* p1) {
  const u32x4 a = *(const u32x4*)p0, b = *(const u32x4*)p1;
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ inline f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(256, Fp8Cfg<D>::OCC) void fwd_fp8_kernel(Fp8FwdArgs a) {
  constexpr int BC = 64;
  constexpr int DC = D / 64;  // 64-wide d chunks of S
  constexpr int DT = D / 32;  // 32-wide d tiles of O^T
  constexpr int TB = 64 * D;  // bytes per K or V^T tile
  using KL = Fp8Tile<D>;
  using VL = Fp8Tile<64>;
  __shared__ __attribute__((aligned(1024))) unsigned char Ks0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Ks1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs1[TB];
  auto kbuf = [&](int p) -> unsigned char* { return p ? Ks1 : Ks0; };
  auto vbuf = [&](int p) -> unsigned char* { return p ? Vs1 : Vs0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int ql = lane & 31;
  const int hh = lane >> 5;

  const int N = a.N;
  const int nqb = (N + 127) / 128;
  const int nkt = (N + 63) / 64;
  const BlockPick pk = pick_block(blockIdx.x, gridDim.x, nqb, a.B * a.H, a.causal, Fp8Cfg<D>::OCC);
  const int bh = pk.bh;
  const int qb = a.causal ? nqb - 1 - pk.rank : pk.rank;
  const int b = bh / a.H;

  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q8 + (size_t)bh * N * D, (uint32_t)N * D);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k8 + (size_t)bh * N * D, (uint32_t)kv_end * D);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.vt8 + (size_t)bh * D * a.Np, (uint32_t)D * a.Np);

  const int q_blk0 = qb * 128;
  const int q_blk_last = min(q_blk0 + 128, N) - 1;
  int kv_lim = kv_end;
  if (a.causal) kv_lim = min(kv_lim, q_blk_last + 1);
  const int ntiles = (kv_lim + BC - 1) / BC;
  const int wq0 = q_blk0 + wave * 32;
  const int my_q = wq0 + ql;
  int w_lim = kv_end;
  if (a.causal) w_lim = min(w_lim, min(wq0 + 31, N - 1) + 1);
  const int w_tiles = (max(w_lim, 0) + BC - 1) / BC;

  // Score scale in log2 units, times the key tile's scale per tile.
  const float f0 = a.scale * kLog2e * a.q_scale[(size_t)bh * nqb + qb] / (a.rotated ? (float)D : 1.f);
  const float* __restrict__ sk = a.k_scale + (size_t)bh * nkt;

  // Q fragment (B operand of S^T): row my_q, bytes [64 dc + 32 hh, +32).
  i32x8 qf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    const u32x4 x0 = buf_load16(rq, (uint32_t)(my_q * D + 64 * dc + 32 * hh));
    const u32x4 x1 = buf_load16(rq, (uint32_t)(my_q * D + 64 * dc + 32 * hh + 16));
    qf[dc] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_ref = -INFINITY;  // running max of the scaled scores, log2 units
  float l_run = 0.f;        // running sum of 256 p over this half's keys

  auto load_k = [&](int j, unsigned char* dst) {
    load_fp8_tile<D, 64>(rk, dst, D, (size_t)j * 64 * D, wave, lane);
  };
  auto load_v = [&](int j, unsigned char* dst) {
    load_fp8_tile<64, D>(rv, dst, a.Np, (size_t)j * 64, wave, lane);
  };

  // Per-lane LDS offsets: K rows kt*32 + ql, chunks 4 dc + 2 hh (+1); V^T
  // rows dt*32 + ql, chunks 2 hh (+1).
  int k_off[2][DC][2], v_off[DT][2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int e = 0; e < 2; ++e) k_off[kt][dc][e] = KL::off(kt * 32 + ql, 4 * dc + 2 * hh + e);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 2; ++e) v_off[dt][e] = VL::off(dt * 32 + ql, 2 * hh + e);

  auto compute_s = [&](const unsigned char* kb, f32x16 (&s)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        s[kt] = mfma8(read32(kb + k_off[kt][dc][0], kb + k_off[kt][dc][1]), qf[dc], s[kt]);
    }
  };

  // The pipeline of the bf16 forward: K two tiles ahead, V one ahead, S of
  // tile j+1 computed while tile j's softmax and P V run.
  f32x16 s_a[2], s_b[2];
  // Key-block scale of the current tile, loaded one tile ahead so that no
  // tile waits for it.
  float sk_cur = 0.f;
  if (ntiles > 0) {
    sk_cur = sk[0];
    load_k(0, Ks0);
    load_k(1, Ks1);
    load_v(0, Vs0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (w_tiles > 0) compute_s(Ks0, s_a);
  }

  // FULL tiles (every row of every wave sees every key of tiles j and j+1)
  // run with no mask and no liveness test, so that S(j+1), the
  // exponentials and the P V products of tile j share one basic block.
  auto tile = [&](int j, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], auto full, int par) {
    constexpr bool FULL = decltype(full)::value;
    // Every wave has finished tile j-1: the K buffer of tile j and the V
    // buffer of tile j-1 are free. Loads past the last tile read inside the
    // head's buffers, or zeros past their end, and are never used.
    __syncthreads();
    if (FULL || j + 2 < ntiles) load_k(j + 2, kbuf(par));
    if (FULL || j + 1 < ntiles) load_v(j + 1, vbuf(par ^ 1));
    const float f = f0 * sk_cur;
    // a wave-uniform index makes this a scalar load, which no vector-memory
    // wait of the tile's copies then covers
    sk_cur = sk[min(__builtin_amdgcn_readfirstlane(j + 1), nkt - 1)];
    if (FULL || j < w_tiles) {
      const int t0 = j * BC;
      const bool need_mask = !FULL && ((t0 + BC > kv_end) || (a.causal && t0 + BC - 1 > wq0));
      // lane = query; register r of sub-tile kt holds key t0 + kt*32 + 8(r/4) + 4hh + r%4
      auto hidden = [&](int kt, int r) {
        const int key = t0 + kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        return key >= kv_end || (a.causal && key > my_q);
      };
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, (need_mask && hidden(kt, r)) ? -INFINITY : s_cur[kt][r]);
      mx = halves_max(mx);
      const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * f;
      if (__any(m_tile > m_ref)) {
        const float m_new = fmaxf(m_ref, m_tile);
        const float alpha = (m_new == m_ref) ? 1.f : fast_exp2(m_ref - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        m_ref = m_new;
      }
      if constexpr (FULL) {
        __builtin_amdgcn_iglp_opt(0);
        __builtin_amdgcn_s_setprio(1);
      }
      if (FULL || j + 1 < w_tiles) compute_s(kbuf(par ^ 1), s_nxt);

      // 256 p = exp2(s f - m + 8); hidden keys and rows with no key yet give 0.
      const float bias = (m_ref == -INFINITY) ? 0.f : 8.f - m_ref;
      float lsum = 0.f;
      unsigned pw[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = fast_exp2(fmaf(s_cur[kt][r], f, bias));
          if (need_mask && hidden(kt, r)) v = 0.f;
          p[r] = v;
          lsum += v;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) pw[kt][g] = pack4(p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]);
      }
      l_run += lsum;
      // Half hh of the wave holds, for each group g of 8 keys, the 4 keys
      // 8g + 4hh .. +3 of both sub-tiles. One swap per g gives the lower half
      // keys 0-31 and the upper half keys 32-63 of the tile, in order: the
      // B operand of P^T with k = key - 32 hh.
      i32x8 pf;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const auto sw = __builtin_amdgcn_permlane32_swap(pw[0][g], pw[1][g], false, false);
        pf[2 * g] = (int)sw[0];
        pf[2 * g + 1] = (int)sw[1];
      }
      const unsigned char* vb = vbuf(par);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma8(read32(vb + v_off[dt][0], vb + v_off[dt][1]), pf, oacc[dt]);
      if constexpr (FULL) __builtin_amdgcn_s_setprio(0);
    }
    // This wave's copies of the next tiles must have landed before anyone
    // passes the next barrier.
    __builtin_amdgcn_s_waitcnt(0);
  };

  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  const int n_vis = (a.causal ? min(kv_end, q_blk0 + 1) : kv_end) / BC;
  const int n_full = max(min(n_vis, ntiles - 1), 0) & ~1;
  int j = 0;
  for (; j < n_full; j += 2) {
    tile(j, s_a, s_b, Full{}, 0);
    tile(j + 1, s_b, s_a, Full{}, 1);
  }
  for (; j < ntiles; ++j) {
    tile(j, s_a, s_b, Part{}, j & 1);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s_a[kt] = s_b[kt];
  }

  // O = acc * scale_v / l (the 256 of P and of l cancel); LSE in natural log.
  const float l_tot = halves_sum(l_run);
  const float inv = (l_tot > 0.f) ? a.v_scale[bh] / l_tot : 0.f;
  if (my_q < N) {
    const size_t head_off = (size_t)bh * N * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + r4 * 8 + 4 * hh;
        const float o0 = oacc[dt][4 * r4 + 0] * inv, o1 = oacc[dt][4 * r4 + 1] * inv;
        const float o2 = oacc[dt][4 * r4 + 2] * inv, o3 = oacc[dt][4 * r4 + 3] * inv;
        if constexpr (OUT_F32) {
          *(f32x4*)((float*)a.o + head_off + (size_t)my_q * D + d0) = f32x4{o0, o1, o2, o3};
        } else {
          uint16_t* Og = (uint16_t*)a.o + head_off + (size_t)my_q * D + d0;
          if (a.o_bf16)
            *(u32x2*)Og = u32x2{Mfma<BF16>::pack(o0, o1), Mfma<BF16>::pack(o2, o3)};
          else
            *(u32x2*)Og = u32x2{Mfma<F16>::pack(o0, o1), Mfma<F16>::pack(o2, o3)};
        }
      }
    }
    if (hh == 0)
      a.lse[(size_t)bh * N + my_q] = (l_tot > 0.f) ? (m_ref + fast_log2(l_tot) - 8.f) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_quant(const Fp8QuantArgs& a, hipStream_t s) {
  const long BH = (long)a.B * a.H;
  const long nq = (a.N + 127) / 128, nk = (a.N + 63) / 64;
  hipLaunchKernelGGL((fp8_qk_kernel<T, D>), dim3((unsigned)(BH * (nq + 2 * nk))), dim3(kQThreads), 0,
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fp8_v_kernel<T, D>), dim3((unsigned)(BH * nk)), dim3(kQThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attn(const Fp8FwdArgs& a, bool of, hipStream_t s) {
  const long nqb = (a.N + 127) / 128;
  const dim3 grid((unsigned)((long)a.B * a.H * nqb));
  if (of) hipLaunchKernelGGL((fwd_fp8_kernel<D, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((fwd_fp8_kernel<D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8QuantArgs& a, Elem in, hipStream_t s) {
  if (in == Elem::BF16) return a.d == 128 ? launch_quant<BF16, 128>(a, s) : launch_quant<BF16, 64>(a, s);
  return a.d == 128 ? launch_quant<F16, 128>(a, s) : launch_quant<F16, 64>(a, s);
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, Elem out, hipStream_t s) {
  const bool of = (out == Elem::F32);
  return a.d == 128 ? launch_attn<128>(a, of, s) : launch_attn<64>(a, of, s);
}

}  // namespace fa
