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
// Two launches, no atomics, so the result is bit-reproducible (a third,
// dsum_kernel, computes D_i = rowsum(dO * O) on its own for callers who want
// that stage alone):
//   2. dkdv_kernel:  one workgroup per key block, after dq_kernel (it reads
//      D from the workspace); K and V stay in VGPRs, the
//      loop streams query tiles (Q, dO from HBM straight into LDS; LSE, D)
//      past them. Per tile: S = Q K^T and dP = dO V^T with the key as the
//      accumulator column (lane), so P and dS come out of the accumulator
//      already in the layout the next two products take as B operand:
//      dV^T += dO^T P, dK^T += Q^T dS, whose A operands (dO^T, Q^T) are
//      transposed reads (ds_read_b64_tr_b16) of the same row-major tiles.
//   1. dq_kernel: one workgroup per query block; it first forms D_i =
//      rowsum(dO * O) for its rows and writes it to the workspace; Q and dO
//      stay in VGPRs, the
//      loop streams key tiles (K, V) through LDS. Per tile: S^T = K Q^T and
//      dP^T = V dO^T with the query as the lane, then dQ^T += K^T dS^T with
//      K^T a transposed read of the K tile.
// The dQ kernel recomputes S and dP, so the MFMA work is 7 products per tile
// pair against the 5 the gradients need.
#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// Eight O values of one row, as fp32: elements [e0, e0 + 8) of the row
// starting at element offset `row_off` of the head (O in the 16-bit type T,
// or fp32 when o_f32).
template <typename T>
struct ORow8 {
  float x[8];
};
template <typename T>
__device__ inline ORow8<T> load_o8(__amdgpu_buffer_rsrc_t r, uint32_t elem_off, bool o_f32) {
  ORow8<T> v;
  if (o_f32) {
    const f32x4 a = __builtin_bit_cast(f32x4, buf_load16(r, elem_off * 4));
    const f32x4 b = __builtin_bit_cast(f32x4, buf_load16(r, elem_off * 4 + 16));
    v.x[0] = a[0];
    v.x[1] = a[1];
    v.x[2] = a[2];
    v.x[3] = a[3];
    v.x[4] = b[0];
    v.x[5] = b[1];
    v.x[6] = b[2];
    v.x[7] = b[3];
  } else {
    const u32x4 a = buf_load16(r, elem_off * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v.x[2 * i] = Mfma<T>::to_f32(a[i] & 0xffffu);
      v.x[2 * i + 1] = Mfma<T>::to_f32(a[i] >> 16);
    }
  }
  return v;
}

// sum_e o[e] * g[e] over one 8-element chunk, in element order, onto acc
// (g: the matching 8 dO values, 16-bit, in a u32x4).
template <typename T>
__device__ inline float dot8(const ORow8<T>& o, u32x4 g, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(o.x[2 * i], Mfma<T>::to_f32(g[i] & 0xffffu), acc);
    acc = fmaf(o.x[2 * i + 1], Mfma<T>::to_f32(g[i] >> 16), acc);
  }
  return acc;
}

// D_i = sum_c dO_ic O_ic (fp32), in the order the dQ kernel forms it (two
// lanes per row; lane h sums the 8-element chunks 16 c + 8 h, c = 0, 1, ...,
// in turn; then the two halves are added), so that D, and a backward run as
// D, dK/dV and dQ stages, equal the one-call backward bit for bit.
template <typename T, int D>
__global__ __launch_bounds__(256) void dsum_kernel(const void* __restrict__ o,
                                                   const uint16_t* __restrict__ dout,
                                                   float* __restrict__ dsum, long rows, int o_f32) {
  constexpr int RPB = 128;  // rows per workgroup
  const int tid = threadIdx.x;
  const long row0 = (long)blockIdx.x * RPB;
  const long row = row0 + tid / 2;
  const int h = tid & 1;
  // this workgroup's rows of O as a buffer (32-bit offsets inside it)
  const long nrows = min((long)RPB, rows - row0);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(
      (const unsigned char*)o + row0 * D * (o_f32 ? 4 : 2), (uint32_t)(nrows * D * (o_f32 ? 4 : 2)));
  float acc = 0.f;
  if (row < rows) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const ORow8<T> ov = load_o8<T>(ro, (uint32_t)((row - row0) * D + c * 16 + h * 8), o_f32 != 0);
      const u32x4 gv = *(const u32x4*)(dout + row * D + c * 16 + h * 8);
      acc = dot8<T>(ov, gv, acc);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  if (row < rows && h == 0) dsum[row] = acc;
}

template <typename T>
__device__ inline u32x4 pack8(const f32x16& x, int base) {
  return u32x4{Mfma<T>::pack(x[base + 0], x[base + 1]), Mfma<T>::pack(x[base + 2], x[base + 3]),
               Mfma<T>::pack(x[base + 4], x[base + 5]), Mfma<T>::pack(x[base + 6], x[base + 7])};
}

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (b, h, key block of 128 keys); wave w owns keys
// [32w, 32w + 32) with their K and V rows in VGPRs. Query tiles of BQ rows
// (Q, dO straight from HBM into LDS, LSE and D through VGPRs) stream past.
template <int D>
struct DkdvCfg {
  static constexpr int BQ = 64;                  // queries per tile
  static constexpr int MINW = (D == 128) ? 1 : 2;  // waves per SIMD the registers allow
  // D = 64: the dP products of a sub-tile start from -D_i instead of 0, so
  // that they yield dP - D directly, and a full tile forms S and dP of both
  // sub-tiles before the exponentials of the first (measured faster at D =
  // 64, slower at D = 128).
  static constexpr bool DP_MINUS_D = (D == 64);
  // D = 64: the query tiles are walked from the last down to the first, so
  // that the key blocks of a head running at the same time read the same Q
  // and dO tile at about the same time and all but the first find it in L2
  // (walked upwards, each key block starts at its own causal diagonal).
  // Measured 3% faster on the GPT-2 shape; at D = 128 the compiler then
  // schedules the LDS reads of the full tiles one product ahead (38% slower).
  // The block-sparse kernel walks the same way, so that an all-kept mask
  // gives the dense result bit for bit (walked upwards it measured 2% faster
  // planned and 9-13% faster unplanned at D = 64).
  static constexpr bool DOWN = (D == 64);
};

// SP: block-sparse, only the query tiles of the query blocks the block mask
// keeps against this key block (no grouped K/V heads).
template <typename T, int D, bool SP>
__global__ __launch_bounds__(kBwdThreads, DkdvCfg<D>::MINW) void dkdv_kernel(BwdArgs a) {
  using L = TileLayout<D>;
  constexpr int BK = 32 * kBwdWaves;  // keys per workgroup
  constexpr int BQ = DkdvCfg<D>::BQ;
  constexpr int QS = BQ / 32;         // 32-query sub-tiles
  constexpr int DC = D / 16;
  constexpr int DT = D / 32;
  constexpr int TB = L::bytes(BQ);

  // Double buffers of Q, dO, LSE (times log2 e) and D as separate variables,
  // so the compiler can tell a copy into one buffer from reads of the other.
  // Query tile it uses the buffers of parity it & 1.
  __shared__ __attribute__((aligned(1024))) unsigned char Qs0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Qs1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Gs0[TB];  // dO
  __shared__ __attribute__((aligned(1024))) unsigned char Gs1[TB];
  __shared__ __attribute__((aligned(16))) float Ls0[BQ];
  __shared__ __attribute__((aligned(16))) float Ls1[BQ];
  __shared__ __attribute__((aligned(16))) float Ds0[BQ];
  __shared__ __attribute__((aligned(16))) float Ds1[BQ];
  auto qbuf = [&](int p) -> unsigned char* { return p ? Qs1 : Qs0; };
  auto gbuf = [&](int p) -> unsigned char* { return p ? Gs1 : Gs0; };
  auto lbuf = [&](int p) -> float* { return p ? Ls1 : Ls0; };
  auto dbuf = [&](int p) -> float* { return p ? Ds1 : Ds0; };
  __shared__ unsigned short blist[SP ? kMaxMaskBlocks + 2 : 1];
  __shared__ int bwc[SP ? kBwdWaves : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int kl = lane & 31;
  const int hh = lane >> 5;

  const int N = a.N;
  const int nkb = (N + BK - 1) / BK;
  // One workgroup per (b, K/V head, query-head share, key block); with
  // grouped K/V heads it runs the tiles of each query head of its share in
  // turn (a share is G / gsplit consecutive heads of the group of G).
  const int S = a.gsplit;
  const BlockPick pk = pick_block(blockIdx.x, gridDim.x, nkb, a.B * a.Hkv * S, a.causal,
                                  DkdvCfg<D>::MINW);
  int bhk = pk.bh / S;  // K/V head
  const int share = pk.bh - bhk * S;
  int kb = pk.rank;  // causal: key block 0 sees every query and has the most work
  // Block-sparse by pieces: the workgroup's item names its column and piece.
  int piece0 = 0, slot = -1;
  const bool by_items = SP && a.sp_items != nullptr;
  if (by_items) {
    const int* it4 = a.sp_items + 4 * (size_t)blockIdx.x;
    bhk = __builtin_amdgcn_readfirstlane(it4[0]);
    kb = __builtin_amdgcn_readfirstlane(it4[1]);
    piece0 = __builtin_amdgcn_readfirstlane(it4[2]);
    slot = __builtin_amdgcn_readfirstlane(it4[3]);
  }
  const int b = bhk / a.Hkv;
  const int G = a.H / a.Hkv;
  const int g0 = share * (G / S), g1 = g0 + G / S;

  const size_t head_off = (size_t)bhk * N * D;  // K, V, dK, dV
  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t*)a.k + head_off, (uint32_t)kv_end * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t*)a.v + head_off, (uint32_t)kv_end * D * 2);
  // Q, dO, LSE and D of the query head being run (set per query head below)
  __amdgpu_buffer_rsrc_t rq, rg;
  const float* __restrict__ Lg;
  const float* __restrict__ Dg;
  auto set_query_head = [&](int g) {
    const size_t bhq = (size_t)b * a.H + (size_t)(bhk - b * a.Hkv) * G + g;
    rq = make_rsrc((const uint16_t*)a.q + bhq * N * D, (uint32_t)N * D * 2);
    rg = make_rsrc((const uint16_t*)a.dout + bhq * N * D, (uint32_t)N * D * 2);
    Lg = a.lse + bhq * N;
    Dg = a.dsum + bhq * N;
  };

  const int key0 = kb * BK + wave * 32;
  const int my_key = key0 + kl;

  // B operands of S = Q K^T and dP = dO V^T: this lane's key row, 8 d
  // elements per 16-wide chunk. Keys at or past kv_end read as zero.
  u32x4 kf[DC], vf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    kf[dc] = buf_load16(rk, (uint32_t)(my_key * D + dc * 16 + hh * 8) * 2);
    vf[dc] = buf_load16(rv, (uint32_t)(my_key * D + dc * 16 + hh * 8) * 2);
  }

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  const int blk_key0 = kb * BK;
  const int qt_begin = (a.causal ? blk_key0 : 0) / BQ;
  const int qt_end = (blk_key0 < kv_end) ? (N + BQ - 1) / BQ : qt_begin;
  const float sl2 = a.scale * kLog2e;

  // Query tiles run as a sequence c in [c_begin, c_end), tile tile_ix(c):
  // all tiles from qt_begin, or (block-sparse) only those of the query
  // blocks kept against this key block, in increasing order.
  int c_begin = qt_begin, c_end = qt_end, n_kept = 0;
  // Block-sparse: the list from this piece's first block on, and that
  // block's tile position in the whole list. A piece counts its tiles from
  // 0 (with the piece's first position as c_begin instead, the compiler
  // issued the full tiles' LDS reads one MFMA ahead).
  const unsigned short* plist = blist;
  int p0 = 0;
  if constexpr (SP) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const unsigned char* mcol = a.bmask + (long long)b * a.bm_sb +
                                (long long)(bhk - b * a.Hkv) * a.bm_sh + kb;
    // BK is the mask block, so qt_begin is even: block qt_begin / 2 starts it.
    n_kept = list_mask_blocks<kBwdThreads>(mcol, nb, qt_begin / 2, (qt_end + 1) / 2, blist, bwc);
    c_begin = 0;
    c_end = mask_tiles_below(blist, n_kept, qt_end);
    if (by_items) {  // this piece: listed blocks [piece0, piece0 + kSparsePiece)
      p0 = 2 * min(piece0, n_kept);
      plist = blist + p0 / 2;
      c_end = max(min(c_end - p0, 2 * kSparsePiece), 0);
    }
  }
  auto tile_ix = [&](int c) -> int {
    if constexpr (SP) return mask_tile(plist, c);
    else return c;
  };

  // Row-major fragment reads (A of S and dP): row qs*32 + kl, chunk 2dc + hh.
  int r_off[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) r_off[dc] = L::off(kl, 2 * dc + hh);
  // Transposed fragment reads (A of dV^T and dK^T): 16 queries x 32 d.
  int t_off[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) t_off[dt] = L::tr_off(lane, dt * 32);

  // LSE and D of a query tile go through one VGPR of the first 2*BQ threads:
  // loaded raw at the start of the previous tile and only used (scaled and
  // stored to LDS) at its end, so that no instruction of that tile waits for
  // the load (loads complete in order, so such a wait would also wait for
  // the tile copies issued just before it). A row without any visible key
  // (LSE = -inf) has all its probabilities masked; a finite stand-in avoids
  // inf - inf.
  float sreg = 0.f;
  auto load_stats = [&](int it) {
    if (tid < 2 * BQ) {
      const int q = it * BQ + (tid % BQ);
      sreg = 0.f;
      if (q < N) sreg = (tid < BQ) ? Lg[q] : Dg[q];
    }
  };
  auto store_stats = [&](int p) {
    if (tid < BQ) lbuf(p)[tid] = (sreg == -INFINITY) ? 0.f : sreg * kLog2e;
    else if (tid < 2 * BQ) dbuf(p)[tid - BQ] = DkdvCfg<D>::DP_MINUS_D ? -sreg : sreg;
  };
  auto load_tiles = [&](int it, int p) {
    load_tile_lds<D, BQ, kBwdWaves>(rq, qbuf(p), it * BQ, wave, lane);
    load_tile_lds<D, BQ, kBwdWaves>(rg, gbuf(p), it * BQ, wave, lane);
  };

  // First tile of the walk and its buffer parity.
  constexpr bool DOWN = DkdvCfg<D>::DOWN;
  auto prologue = [&]() {
    if (c_begin < c_end) {
      const int c0 = DOWN ? c_end - 1 : c_begin;
      load_tiles(tile_ix(c0), DOWN ? 0 : c_begin & 1);
      load_stats(tile_ix(c0));
      store_stats(DOWN ? 0 : c_begin & 1);
    }
    // Unconditional, so that on every path into the loops below the K and
    // V fragment loads above are known complete: the compiler places waits
    // path by path, and would otherwise wait for them inside every tile,
    // which at run time also waits for that tile's own prefetch copies.
    __builtin_amdgcn_s_waitcnt(0);
  };

  // One query tile. FULL tiles (every key of the workgroup visible to every
  // query of the tile) run with no liveness test and no mask, so both query
  // sub-tiles sit in one basic block. Queries past N need no mask anywhere:
  // their Q and dO rows read as zero and their LSE and D as zero, so their P
  // meets a zero dO row and their dS is zero.
  auto tile = [&](int c, auto full, int buf) {
    constexpr bool FULL = decltype(full)::value;
    // Tile c has landed everywhere; every wave is done with the tile before
    // it in the walk, so the other buffers are free for the one after.
    __syncthreads();
    const bool more = DOWN ? c > c_begin : c + 1 < c_end;
    if (more) {
      const int nxt = tile_ix(DOWN ? c - 1 : c + 1);
      load_tiles(nxt, buf ^ 1);
      load_stats(nxt);
    }
    const int q0 = tile_ix(c) * BQ;
    const bool live = FULL || ((key0 < kv_end) && (!a.causal || q0 + BQ - 1 >= key0));
    // S = Q K^T and dP = dO V^T of query sub-tile qs (32 queries by this
    // wave's 32 keys): lane = key; register r holds query qs*32 + 8(r/4) +
    // 4hh + r%4.
    auto sdp = [&](int qs, f32x16& s, f32x16& dp) {
      const unsigned char* qt = qbuf(buf) + qs * (32 / L::RPI) * L::GB;
      const unsigned char* gt = gbuf(buf) + qs * (32 / L::RPI) * L::GB;
      s = f32x16{};
      if constexpr (DkdvCfg<D>::DP_MINUS_D) {
        // -D_i of each query, as stored in LDS
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 d4 = *(const f32x4*)&dbuf(buf)[qs * 32 + 8 * r4 + 4 * hh];
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * r4 + e] = d4[e];
        }
      } else {
        dp = f32x16{};
      }
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) s = Mfma<T>::mma32(*(const u32x4*)(qt + r_off[dc]), kf[dc], s);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) dp = Mfma<T>::mma32(*(const u32x4*)(gt + r_off[dc]), vf[dc], dp);
    };
    // In place: s becomes P = exp(S - LSE), dp becomes dS = P (dP - D).
    auto probs = [&](int qs, f32x16& s, f32x16& dp, bool need_mask) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qi = qs * 32 + 8 * r4 + 4 * hh;
        const f32x4 l4 = *(const f32x4*)&lbuf(buf)[qi];
        const f32x4 d4 = *(const f32x4*)&dbuf(buf)[qi];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          float p = fast_exp2(fmaf(s[r], sl2, -l4[e]));
          if (need_mask) {
            const int q = q0 + qi + e;
            const bool vis = (my_key < kv_end) && (!a.causal || my_key <= q);
            p = vis ? p : 0.f;
          }
          s[r] = p;
          if constexpr (DkdvCfg<D>::DP_MINUS_D) dp[r] = p * dp[r];
          else dp[r] = p * (dp[r] - d4[e]);
        }
      }
    };
    // dV^T += dO^T P^T and dK^T += Q^T dS^T over the sub-tile's 32 queries.
    auto grads = [&](int qs, const f32x16& s, const f32x16& dp) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 pf = pack8<T>(s, 8 * c2);
        const u32x4 sf = pack8<T>(dp, 8 * c2);
        const int rb = (2 * qs + c2) * L::rows16();
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const unsigned char* gp = gbuf(buf) + rb + t_off[dt];
          const u32x2 g0 = lds_read_tr(gp), g1 = lds_read_tr(gp + L::half_step());
          dv[dt] = Mfma<T>::mma32(u32x4{g0.x, g0.y, g1.x, g1.y}, pf, dv[dt]);
          const unsigned char* qp = qbuf(buf) + rb + t_off[dt];
          const u32x2 q0v = lds_read_tr(qp), q1v = lds_read_tr(qp + L::half_step());
          dk[dt] = Mfma<T>::mma32(u32x4{q0v.x, q0v.y, q1v.x, q1v.y}, sf, dk[dt]);
        }
      }
    };
    if (live) {
      // Full tiles: let the scheduler interleave the four MFMA chains with
      // the exponentials and LDS reads (iglp_opt strategy 0).
      if constexpr (FULL) __builtin_amdgcn_iglp_opt(0);
      const bool need_mask = !FULL && ((key0 + 32 > kv_end) || (a.causal && key0 + 31 > q0));
      if constexpr (FULL && DkdvCfg<D>::DP_MINUS_D) {
        f32x16 s[QS], dp[QS];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) sdp(qs, s[qs], dp[qs]);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          probs(qs, s[qs], dp[qs], false);
          grads(qs, s[qs], dp[qs]);
        }
      } else {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          f32x16 s, dp;
          sdp(qs, s, dp);
          probs(qs, s, dp, need_mask);
          grads(qs, s, dp);
        }
      }
    }
    if (more) store_stats(buf ^ 1);
    __builtin_amdgcn_s_waitcnt(0);
  };

  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  // Tiles from it_full on see every key of the block: the keys all lie below
  // kv_end and (causal) the tile's first query is at or past the last key.
  int it_full = qt_end;
  if (blk_key0 + BK <= kv_end) it_full = a.causal ? max(qt_begin, (blk_key0 + BK - 1 + BQ - 1) / BQ) : qt_begin;
  it_full = min(it_full, qt_end);
  int c_full = it_full;  // sequence position of the first full tile
  if constexpr (SP) c_full = min(max(mask_tiles_below(blist, n_kept, it_full) - p0, c_begin), c_end);
  for (int g = g0; g < g1; ++g) {
    set_query_head(g);
    // Every wave is done with the previous query head's last tile before
    // this head's first tile is copied into the buffers.
    if (g > g0) __syncthreads();
    prologue();
    if constexpr (DOWN) {
      // Step k runs tile c_end - 1 - k in the buffers of parity k & 1: the
      // full tiles first, in pairs of known parity, then the partial ones
      // (the causal diagonal, keys past kv_end).
      const int n_full = c_end - max(c_full, c_begin);
      int k = 0;
      for (; k + 1 < n_full; k += 2) {
        tile(c_end - 1 - k, Full{}, 0);
        tile(c_end - 2 - k, Full{}, 1);
      }
      if (k < n_full) tile(c_end - 1 - k++, Full{}, 0);
      for (; k < c_end - c_begin; ++k) tile(c_end - 1 - k, Part{}, k & 1);
    } else {
      int c = c_begin;
      for (; c < c_full; ++c) tile(c, Part{}, c & 1);
      // Full tiles in pairs of known parity (an odd first tile on its own).
      if (c < c_end && (c & 1)) tile(c++, Full{}, 1);
      for (; c + 1 < c_end; c += 2) {
        tile(c, Full{}, 0);
        tile(c + 1, Full{}, 1);
      }
      if (c < c_end) tile(c, Full{}, 0);
    }
  }

  // dK^T / dV^T accumulators: lane = key, registers = d in runs of 4.
  if (by_items && slot >= 0) {
    // fp32 partials of this piece, rows = keys of the block
    const size_t blk = (size_t)kMaskBlock * D;
    float* dKp = a.dkv_part + (size_t)slot * blk + (size_t)(wave * 32 + kl) * D;
    float* dVp = dKp + (size_t)a.sp_nslots * blk;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + r4 * 8 + 4 * hh;
        const f32x16& K4 = dk[dt];
        const f32x16& V4 = dv[dt];
        *(f32x4*)(dKp + d0) = f32x4{K4[4 * r4] * a.scale, K4[4 * r4 + 1] * a.scale,
                                    K4[4 * r4 + 2] * a.scale, K4[4 * r4 + 3] * a.scale};
        *(f32x4*)(dVp + d0) = f32x4{V4[4 * r4], V4[4 * r4 + 1], V4[4 * r4 + 2], V4[4 * r4 + 3]};
      }
    }
  } else if (S > 1) {
    // fp32 partials of this share; the reduction adds the shares in order.
    if (my_key < N) {
      const size_t part = (size_t)a.B * a.Hkv * N * D;
      float* dKp = a.dkv_part + share * part + head_off + (size_t)my_key * D;
      float* dVp = dKp + (size_t)S * part;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = dt * 32 + r4 * 8 + 4 * hh;
          const f32x16& K4 = dk[dt];
          const f32x16& V4 = dv[dt];
          *(f32x4*)(dKp + d0) = f32x4{K4[4 * r4] * a.scale, K4[4 * r4 + 1] * a.scale,
                                      K4[4 * r4 + 2] * a.scale, K4[4 * r4 + 3] * a.scale};
          *(f32x4*)(dVp + d0) = f32x4{V4[4 * r4], V4[4 * r4 + 1], V4[4 * r4 + 2], V4[4 * r4 + 3]};
        }
      }
    }
  } else {
    // Wave w stages its 32 keys of dK and dV in one of the four query-tile
    // buffers, free once every wave is past its last tile.
    constexpr int SB = L::bytes(32);
    static_assert(2 * SB <= TB, "dK and dV of a wave fit one tile buffer");
    unsigned char* stage = wave == 0 ? Qs0 : wave == 1 ? Qs1 : wave == 2 ? Gs0 : Gs1;
    __syncthreads();
    stage_put<T, D>(stage, dk, a.scale, lane);
    stage_put<T, D>(stage + SB, dv, 1.f, lane);
    __syncthreads();
    stage_rows_out<D>(stage, (uint16_t*)a.dk + head_off + (size_t)key0 * D, N - key0, lane);
    stage_rows_out<D>(stage + SB, (uint16_t*)a.dv + head_off + (size_t)key0 * D, N - key0, lane);
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, h, query block of 128 rows); wave w owns rows
// [32w, 32w + 32) with its Q and dO rows in VGPRs. Key tiles of BC keys (K,
// V straight from HBM into LDS) stream past; K is read both row-wise (A of
// S^T) and transposed (A of dQ^T). Tiles of 64 keys, double-buffered; the
// next tile's loads are in flight while the current one is computed.
// (Computing S/dP of the next tile alongside the current one was measured
// slower than three waves per SIMD without it, at d = 64.)
//
// Rows past N need no mask: their Q and dO rows read as zero and nothing of
// them is stored. Keys past kv_len (or past N) do: their K and V rows read
// as zero, so s = 0 and p = exp(-LSE), which overflows for a very negative
// LSE (fp16 already past 65504 when packing dS); 0 * inf in the dQ product
// would then be NaN. Such keys lie only in the last tile, which is never a
// full tile, so the mask costs the main loop nothing.
template <int D>
struct DqCfg {
  static constexpr int BC = 64;                    // keys per tile
  static constexpr int MINW = (D == 64) ? 3 : 2;  // waves per SIMD the registers allow
};

// SP: block-sparse, only the key tiles of the key blocks the block mask
// keeps for this query block.
template <typename T, int D, bool SP>
__global__ __launch_bounds__(kBwdThreads, DqCfg<D>::MINW) void dq_kernel(BwdArgs a) {
  using L = TileLayout<D>;
  constexpr int BR = 32 * kBwdWaves;
  constexpr int BC = DqCfg<D>::BC;
  constexpr int KT = BC / 32;
  constexpr int DC = D / 16;
  constexpr int DT = D / 32;
  constexpr int TB = L::bytes(BC);

  // Double buffers of K and V as separate variables (see the dK/dV kernel);
  // key tile j uses the buffers of parity j & 1.
  __shared__ __attribute__((aligned(1024))) unsigned char Ks0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Ks1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs1[TB];
  auto kbuf = [&](int p) -> unsigned char* { return p ? Ks1 : Ks0; };
  auto vbuf = [&](int p) -> unsigned char* { return p ? Vs1 : Vs0; };
  __shared__ unsigned short blist[SP ? kMaxMaskBlocks + 2 : 1];
  __shared__ int bwc[SP ? kBwdWaves : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int ql = lane & 31;
  const int hh = lane >> 5;

  const int N = a.N;
  const int nqb = (N + BR - 1) / BR;
  const BlockPick pk = pick_block(blockIdx.x, gridDim.x, nqb, a.B * a.H, a.causal, DqCfg<D>::MINW);
  int bh = pk.bh;
  int qb = a.causal ? nqb - 1 - pk.rank : pk.rank;
  // Block-sparse by row pieces: the workgroup's item names its row and piece.
  int piece0 = 0, slot = -1;
  const bool by_items = SP && a.sq_items != nullptr;
  if (by_items) {
    const int* it4 = a.sq_items + 4 * (size_t)blockIdx.x;
    bh = __builtin_amdgcn_readfirstlane(it4[0]);
    qb = __builtin_amdgcn_readfirstlane(it4[1]);
    piece0 = __builtin_amdgcn_readfirstlane(it4[2]);
    slot = __builtin_amdgcn_readfirstlane(it4[3]);
  }
  const int b = bh / a.H;

  const size_t head_off = (size_t)bh * N * D;
  int kv_end = N;
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), N);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)a.q + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc((const uint16_t*)a.dout + head_off, (uint32_t)N * D * 2);
  // K/V head of this query head (grouped K/V heads share one among H / Hkv)
  const size_t kv_off = (size_t)(b * a.Hkv + (bh - b * a.H) / (a.H / a.Hkv)) * N * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t*)a.k + kv_off, (uint32_t)kv_end * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t*)a.v + kv_off, (uint32_t)kv_end * D * 2);

  const int q_blk0 = qb * BR;
  int kv_lim = kv_end;
  if (a.causal) kv_lim = min(kv_lim, min(q_blk0 + BR, N));
  int ntiles = (kv_lim + BC - 1) / BC;

  const int wq0 = q_blk0 + wave * 32;
  const int my_q = wq0 + ql;
  int w_lim = kv_end;
  if (a.causal) w_lim = min(w_lim, min(wq0 + 31, N - 1) + 1);
  int w_tiles = (w_lim + BC - 1) / BC;

  // Block-sparse: tile counts and positions j count only the tiles of the
  // kept key blocks, in increasing order; tile_ix(j) is the key tile. A row
  // piece sees the list from its first block on, at most kSparsePiece blocks.
  int n_kept = 0;
  const unsigned short* plist = blist;
  if constexpr (SP) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const unsigned char* mrow = a.bmask + (long long)b * a.bm_sb +
                                (long long)(bh - b * a.H) * a.bm_sh + (long long)qb * nb;
    n_kept = list_mask_blocks<kBwdThreads>(mrow, 1, 0, min(nb, (kv_lim + kMaskBlock - 1) / kMaskBlock),
                                           blist, bwc);
    if (by_items) {
      plist = blist + min(piece0, n_kept);
      n_kept = max(min(n_kept - piece0, kSparsePiece), 0);
    }
    w_tiles = mask_tiles_below(plist, n_kept, w_tiles);
    ntiles = mask_tiles_below(plist, n_kept, ntiles);
  }
  auto tile_ix = [&](int j) -> int {
    if constexpr (SP) return mask_tile(plist, j);
    else return j;
  };

  u32x4 qf[DC], gf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    qf[dc] = buf_load16(rq, (uint32_t)(my_q * D + dc * 16 + hh * 8) * 2);
    gf[dc] = buf_load16(rg, (uint32_t)(my_q * D + dc * 16 + hh * 8) * 2);
  }
  auto load_k = [&](int j, int p) {
    load_tile_lds<D, BC, kBwdWaves>(rk, kbuf(p), tile_ix(j) * BC, wave, lane);
  };
  auto load_v = [&](int j, int p) {
    load_tile_lds<D, BC, kBwdWaves>(rv, vbuf(p), tile_ix(j) * BC, wave, lane);
  };
  // The first K/V tile and this row's LSE are fetched now, so that their
  // latency overlaps the loads of O below (issued after the store of D, the
  // copies would wait for it: the compiler keeps memory operations in order
  // around a store it cannot tell apart).
  if (ntiles > 0) {
    load_k(0, 0);
    load_v(0, 0);
  }
  const float l_raw = (my_q < N) ? a.lse[(size_t)bh * N + my_q] : 0.f;
  // D_i = sum_c dO_ic O_ic for this lane's row, from the dO fragments
  // already in VGPRs and the matching O fragments (this half of the wave
  // holds half of the row; the halves are summed). Written to the workspace
  // for the dK/dV kernel, which runs after this one.
  const int ob = a.o_f32 ? 4 : 2;  // bytes per O element
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc((const unsigned char*)a.o + head_off * ob, (uint32_t)N * D * ob);
  float dsum = 0.f;
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    const ORow8<T> of = load_o8<T>(ro, (uint32_t)(my_q * D + dc * 16 + hh * 8), a.o_f32 != 0);
    dsum = dot8<T>(of, gf[dc], dsum);
  }
  dsum = halves_sum(dsum);
  // A wave whose rows see one key tile in all forms D_i exactly from that
  // tile instead, as sum_j P_ij dP_ij over the P and dP it computes (the
  // definition of D that rowsum(dO * O) equals in exact arithmetic), so
  // that O's rounding, which the stored O carries, does not enter dS =
  // P (dP - D). On rows of one or two visible keys that difference is of
  // nearly equal terms and O's rounding would dominate it. Not for rows cut
  // into pieces (a piece sees only part of the row).
  // Tiles that no row of the workgroup sees only partly (causal) form the
  // main loop; a full tile also loads the next one unconditionally, so it
  // must not be the last.
  int n_full = a.causal ? (q_blk0 + 1) / BC : ntiles;
  if constexpr (SP) {
    if (a.causal) n_full = mask_tiles_below(plist, n_kept, n_full);
  }
  n_full = min(n_full, ntiles - 1);
  // (a wave with one tile runs it as a partial tile: n_full is then 0; a
  // row item with slot < 0 is a whole row, not cut)
  const bool whole_row = !by_items || slot < 0;
  const bool single = (w_tiles == 1) && whole_row && n_full <= 0;
  float lse2 = 0.f;
  if (my_q < N) {
    lse2 = (l_raw == -INFINITY) ? 0.f : l_raw * kLog2e;
    // every piece of a row forms the same D_i; the first one stores it
    if (hh == 0 && piece0 == 0 && !single) a.dsum[(size_t)bh * N + my_q] = dsum;
  }
  const float sl2 = a.scale * kLog2e;

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};

  int r_off[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) r_off[dc] = L::off(ql, 2 * dc + hh);
  int t_off[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) t_off[dt] = L::tr_off(lane, dt * 32);

  // The dP products start from -D_i (dp0) instead of 0, so they yield
  // dP - D and dS = P (dP - D) is one multiply per element: 64 fewer VALU
  // instructions per two full tiles.
  auto compute_sdp = [&](int p, f32x16 (&s)[KT], f32x16 (&dp)[KT], float dp0) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const unsigned char* kp = kbuf(p) + kt * (32 / L::RPI) * L::GB;
      const unsigned char* vp = vbuf(p) + kt * (32 / L::RPI) * L::GB;
      s[kt] = f32x16{};
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[kt][r] = dp0;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) s[kt] = Mfma<T>::mma32(*(const u32x4*)(kp + r_off[dc]), qf[dc], s[kt]);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) dp[kt] = Mfma<T>::mma32(*(const u32x4*)(vp + r_off[dc]), gf[dc], dp[kt]);
    }
  };

  if (ntiles > 0) __builtin_amdgcn_s_waitcnt(0);
  // Waves whose rows see one tile: D_i = sum_j P_ij dP_ij over that tile
  // (see `single`), from the same S and dP the tile pass recomputes bit for
  // bit. Only workgroups of at most two tiles can hold such a wave, so the
  // extra barrier is confined to them.
  if (ntiles > 0 && ntiles <= 2 && whole_row) {
    __syncthreads();
    if (single) {
      f32x16 s0[KT], dp0[KT];
      compute_sdp(0, s0, dp0, 0.f);
      const int t0 = tile_ix(0) * BC;
      float acc = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s0[kt][r], sl2, -lse2));
          const int key = t0 + kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          acc = fmaf((key < kv_end && (!a.causal || key <= my_q)) ? p : 0.f, dp0[kt][r], acc);
        }
      }
      dsum = halves_sum(acc);
      if (hh == 0 && my_q < N) a.dsum[(size_t)bh * N + my_q] = dsum;
    }
  }

  // Tile j: S^T/dP^T, then dS and dQ. Full tiles (no causal mask for any
  // row of the workgroup) run with no liveness test.
  auto tile = [&](int j, auto full, int par) {
    constexpr bool FULL = decltype(full)::value;
    // Every wave is done with tile j-1, so its buffers take tile j+1.
    __syncthreads();
    if (FULL || j + 1 < ntiles) {
      load_k(j + 1, par ^ 1);
      load_v(j + 1, par ^ 1);
    }
    if (FULL || j < w_tiles) {
      // Full tiles: raise this wave's issue priority while it runs its MFMA
      // chains, so the SIMD's other waves fill the gaps around them.
      if constexpr (FULL) __builtin_amdgcn_s_setprio(1);
      // Full tiles: the compiler's interleave schedules, exponential
      // interleave (strategy 2) at d = 64 and strategy 1 at d = 128. With the
      // -D start of the dP chains these keep the LDS reads ahead of the
      // products; at d = 128 the default schedule then waited for each read
      // before its product.
      if constexpr (FULL && D == 64) __builtin_amdgcn_iglp_opt(2);
      if constexpr (FULL && D == 128) __builtin_amdgcn_iglp_opt(1);
      f32x16 s_cur[KT], p_cur[KT];
      compute_sdp(par, s_cur, p_cur, -dsum);
      const int t0 = tile_ix(j) * BC;
      const bool need_mask = !FULL && ((t0 + BC > kv_end) || (a.causal && t0 + BC - 1 > wq0));
      // Value r of sub-tile kt is key t0 + 4 hh + c with c = 32 kt + 8 (r / 4)
      // + r % 4 a constant, visible iff the key is at most
      // min(kv_end - 1, my_q): one compare with a per-lane bound per value.
      int lim = kv_end - 1;
      if (a.causal) lim = min(lim, my_q);
      lim -= t0 + 4 * hh;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(s_cur[kt][r], sl2, -lse2));
          if (need_mask) p = (kt * 32 + 8 * (r >> 2) + (r & 3) <= lim) ? p : 0.f;
          p_cur[kt][r] = p * p_cur[kt][r];
        }
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const u32x4 sf = pack8<T>(p_cur[kt], 8 * c2);
          const int rb = (2 * kt + c2) * L::rows16();
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const unsigned char* kp = kbuf(par) + rb + t_off[dt];
            const u32x2 k0 = lds_read_tr(kp), k1 = lds_read_tr(kp + L::half_step());
            dq[dt] = Mfma<T>::mma32(u32x4{k0.x, k0.y, k1.x, k1.y}, sf, dq[dt]);
          }
        }
      }
      if constexpr (FULL) __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
  };

  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  int j = 0;
  for (; j + 1 < n_full; j += 2) {
    tile(j, Full{}, 0);
    tile(j + 1, Full{}, 1);
  }
  for (; j < n_full; ++j) tile(j, Full{}, j & 1);
  for (; j < ntiles; ++j) tile(j, Part{}, j & 1);

  if (by_items && slot >= 0) {
    // fp32 partial dQ of this piece, rows = queries of the block
    float* dQp = a.sq_part + ((size_t)slot * kMaskBlock + wave * 32 + ql) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + r4 * 8 + 4 * hh;
        const f32x16& Q4 = dq[dt];
        *(f32x4*)(dQp + d0) = f32x4{Q4[4 * r4] * a.scale, Q4[4 * r4 + 1] * a.scale,
                                    Q4[4 * r4 + 2] * a.scale, Q4[4 * r4 + 3] * a.scale};
      }
    }
  } else {
    // dQ of the wave's 32 rows through LDS (every wave is past its last
    // tile, so the K and V buffers are free) and out in whole rows. The
    // staging costs the kernel about 2 us on the GPT-2 shape, and saves
    // about 3 us of the gap before the next kernel.
    unsigned char* stage = wave == 0 ? Ks0 : wave == 1 ? Ks1 : wave == 2 ? Vs0 : Vs1;
    __syncthreads();
    stage_put<T, D>(stage, dq, a.scale, lane);
    __syncthreads();
    stage_rows_out<D>(stage, (uint16_t*)a.dq + head_off + (size_t)wq0 * D, N - wq0, lane);
  }
}

// dK, dV = the sum of the S fp32 partials of the grouped dK/dV stage, in
// share order, rounded once to the storage type. HBM-bound: per element
// 4 * S bytes read, 2 written. n4 = elements per tensor / 4.
template <typename T>
__global__ __launch_bounds__(256) void dkv_reduce_kernel(const float* __restrict__ part,
                                                         uint16_t* __restrict__ dk,
                                                         uint16_t* __restrict__ dv, long long n4,
                                                         int S) {
  const long long step = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n4; i += step) {
    const int t = i >= n4;  // 0: dK, 1: dV
    const long long j = i - t * n4;
    const f32x4* p = (const f32x4*)part + (long long)t * S * n4 + j;
    f32x4 acc = p[0];
    for (int sh = 1; sh < S; ++sh) {
      const f32x4 x = p[sh * n4];
      acc[0] += x[0];
      acc[1] += x[1];
      acc[2] += x[2];
      acc[3] += x[3];
    }
    uint16_t* out = (t ? dv : dk) + 4 * j;
    *(u32x2*)out = u32x2{Mfma<T>::pack(acc[0], acc[1]), Mfma<T>::pack(acc[2], acc[3])};
  }
}

// dK, dV of the block-sparse columns cut into pieces: the sum of each
// column's fp32 piece partials, in piece order, rounded once. One wave per
// (column, 256 / D key rows), so that even a few cut columns spread over
// the chip; thread t covers 4 consecutive elements.
template <typename T, int D>
__global__ __launch_bounds__(kReduceThreads) void sparse_dkv_reduce_kernel(BwdArgs a) {
  constexpr int ROWS = kReduceThreads * 4 / D;  // key rows per workgroup (4 or 2)
  const int col = blockIdx.x / (kMaskBlock / ROWS);
  const int r0 = (blockIdx.x % (kMaskBlock / ROWS)) * ROWS;
  const int* c4 = a.sp_cols + 4 * (size_t)col;
  const int bh = c4[0], kb = c4[1], slot0 = c4[2], np = c4[3];
  const int e = threadIdx.x * 4;               // element within ROWS x D
  const int row = r0 + e / D, d0 = e % D;
  const int key = kb * kMaskBlock + row;
  if (key >= a.N) return;
  const size_t blk = (size_t)kMaskBlock * D;
  const float* pk = a.dkv_part + (size_t)slot0 * blk + (size_t)row * D + d0;
  const float* pv = pk + (size_t)a.sp_nslots * blk;
  f32x4 sk = *(const f32x4*)pk, sv = *(const f32x4*)pv;
#pragma unroll 4
  for (int i = 1; i < np; ++i) {
    const f32x4 xk = *(const f32x4*)(pk + i * blk), xv = *(const f32x4*)(pv + i * blk);
    sk[0] += xk[0]; sk[1] += xk[1]; sk[2] += xk[2]; sk[3] += xk[3];
    sv[0] += xv[0]; sv[1] += xv[1]; sv[2] += xv[2]; sv[3] += xv[3];
  }
  const size_t off = ((size_t)bh * a.N + key) * D + d0;
  *(u32x2*)((uint16_t*)a.dk + off) = u32x2{Mfma<T>::pack(sk[0], sk[1]), Mfma<T>::pack(sk[2], sk[3])};
  *(u32x2*)((uint16_t*)a.dv + off) = u32x2{Mfma<T>::pack(sv[0], sv[1]), Mfma<T>::pack(sv[2], sv[3])};
}

// dQ of the block-sparse rows cut into pieces: the pieces' fp32 partials
// added in piece order and rounded once.
template <typename T, int D>
__global__ __launch_bounds__(kReduceThreads) void sparse_dq_reduce_kernel(BwdArgs a) {
  constexpr int ROWS = kReduceThreads * 4 / D;
  const int row = blockIdx.x / (kMaskBlock / ROWS);
  const int r0 = (blockIdx.x % (kMaskBlock / ROWS)) * ROWS;
  const int* c4 = a.sq_rows + 4 * (size_t)row;
  const int bh = c4[0], qb = c4[1], slot0 = c4[2], np = c4[3];
  const int e = threadIdx.x * 4;
  const int r = r0 + e / D, d0 = e % D;
  const int q = qb * kMaskBlock + r;
  if (q >= a.N) return;
  const size_t blk = (size_t)kMaskBlock * D;
  const float* p = a.sq_part + (size_t)slot0 * blk + (size_t)r * D + d0;
  f32x4 acc = *(const f32x4*)p;
#pragma unroll 4
  for (int i = 1; i < np; ++i) {
    const f32x4 x = *(const f32x4*)(p + i * blk);
    acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
  }
  *(u32x2*)((uint16_t*)a.dq + ((size_t)bh * a.N + q) * D + d0) =
      u32x2{Mfma<T>::pack(acc[0], acc[1]), Mfma<T>::pack(acc[2], acc[3])};
}

template <typename T, int D, bool SP = false>
hipError_t launch(const BwdArgs& a, int stages, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (stages & (int)BwdStage::DSUM) {
    const long rows = (long)a.B * a.H * a.N;
    constexpr int RPB = 128;
    hipLaunchKernelGGL((dsum_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       st, a.o, (const uint16_t*)a.dout, a.dsum, rows, a.o_f32);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & (int)BwdStage::DQ) {
    const long nqb = (a.N + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
    const long grid = (SP && a.sq_items) ? (long)a.sq_nitems : (long)a.B * a.H * nqb;
    hipLaunchKernelGGL((dq_kernel<T, D, SP>), dim3((unsigned)grid), dim3(kBwdThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (SP && a.sq_items && a.sq_nrows > 0) {
      hipLaunchKernelGGL((sparse_dq_reduce_kernel<T, D>),
                         dim3((unsigned)((long)a.sq_nrows * (kMaskBlock / (kReduceThreads * 4 / D)))),
                         dim3(kReduceThreads), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (stages & (int)BwdStage::DKDV) {
    const long nkb = (a.N + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
    const long grid = (SP && a.sp_items) ? (long)a.sp_nitems : (long)a.B * a.Hkv * a.gsplit * nkb;
    hipLaunchKernelGGL((dkdv_kernel<T, D, SP>), dim3((unsigned)grid), dim3(kBwdThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (SP && a.sp_items && a.sp_ncols > 0) {
      hipLaunchKernelGGL((sparse_dkv_reduce_kernel<T, D>),
                         dim3((unsigned)((long)a.sp_ncols * (kMaskBlock / (kReduceThreads * 4 / D)))),
                         dim3(kReduceThreads), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.gsplit > 1) {
      const long long n4 = (long long)a.B * a.Hkv * a.N * D / 4;
      const long long blocks = (2 * n4 + 255) / 256 < 8192 ? (2 * n4 + 255) / 256 : 8192;
      hipLaunchKernelGGL((dkv_reduce_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, st,
                         a.dkv_part, (uint16_t*)a.dk, (uint16_t*)a.dv, n4, a.gsplit);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return e;
}

template <typename T, bool SP = false>
hipError_t launch_t(const BwdArgs& a, int stages, hipStream_t st) {
  return (a.d == 128) ? launch<T, 128, SP>(a, stages, st) : launch<T, 64, SP>(a, stages, st);
}

}  // namespace

int bwd_group_split(int B, int H, int Hkv, int N, int d) {
  const int G = H / Hkv;
  const long long nkb = (N + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
  const long long slots = 8LL * kCusPerXcd * (d == 128 ? DkdvCfg<128>::MINW : DkdvCfg<64>::MINW);
  const long long base = (long long)B * Hkv * nkb;
  for (int s = 1; s < G; ++s)
    if (G % s == 0 && base * s >= 2 * slots) return s;
  return G;
}

hipError_t launch_bwd_mfma(const BwdArgs& a, Elem t, int stages, hipStream_t st) {
  return (t == Elem::BF16) ? launch_t<BF16>(a, stages, st) : launch_t<F16>(a, stages, st);
}

hipError_t launch_bwd_mfma_sparse(const BwdArgs& a, Elem t, int stages, hipStream_t st) {
  const int s = stages & ((int)BwdStage::DQ | (int)BwdStage::DKDV);
  return (t == Elem::BF16) ? launch_t<BF16, true>(a, s, st) : launch_t<F16, true>(a, s, st);
}

}  // namespace fa
