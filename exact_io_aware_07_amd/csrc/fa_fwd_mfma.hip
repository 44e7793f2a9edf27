// Forward exact attention for bf16 / fp16 inputs on gfx950 MFMA.
//
// The method: split Q into row blocks and K, V into column blocks; for each
// query block stream every key/value block through on-chip memory, keep a
// running row max m and row sum l, rescale the partial output by
// exp(m_old - m_new) when the max grows, and divide by l once at the end
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
//  * S^T = K Q^T on v_mfma_f32_32x32x16 (A = 32 keys of the K tile in LDS,
//    B = the wave's Q rows, resident in VGPRs). In the 32x32 accumulator
//    lane l holds query l % 32 and 16 keys, so a row's max and sum are
//    in-lane plus one exchange with lane l ^ 32 (v_permlane32_swap).
//  * O^T += V^T P^T on the same MFMA. P leaves the S accumulator already in
//    B-operand order (lane = query, keys in runs of 4). V stays row-major in
//    LDS; ds_read_b64_tr_b16 hands each lane 4 consecutive keys of one d
//    column, which is exactly the A-operand order that matches P.
//  * Software pipeline: while tile j's softmax and P V run, S for tile j+1 is
//    already being computed from the next K tile, so the MFMA unit has
//    independent work during the exponentials. K tiles run one tile ahead of
//    V tiles through two LDS buffers each; one barrier per tile.
//  * K and V tiles go from HBM straight into LDS (buffer_load ... lds), no
//    VGPR staging: each load instruction fills 1 KiB of LDS (4 rows at
//    d = 128, 8 at d = 64); those 1 KiB groups are padded by 16 bytes and the
//    16-byte chunks of a row are XOR-swizzled by the row's place in its group,
//    so the K fragment reads (32 rows, one chunk) and the transposed V reads
//    (4 rows, two chunks per 16 lanes) hit distinct LDS banks.
//  * Global loads use buffer resources whose size ends at the last visible
//    key, so rows past the end read as zero with no branch.
//  * Scores stay in raw units; exp2(s * scale * log2 e - m * scale * log2 e)
//    is one FMA and one v_exp_f32 per score.
//  * The running max is exact, so the largest probability of a row is
//    exactly 1 and is not rounded when P is cast for the P V product (a
//    stale reference would put the dominant key's probability at an
//    arbitrary value and round it, which matters when one key dominates a
//    row). The rescale of O is skipped, wave-uniformly, when no row max of
//    the wave moved.
#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;  // query rows per workgroup

template <int D>
struct FwdTile {
  static constexpr int BC = 64;                    // keys per tile
  static constexpr int OCC = (D == 64) ? 3 : 2;  // waves per SIMD the registers allow
};

// GEN: the general form (key count, positions and key split from the
// arguments); without it they are folded to the plain forward's (Nk = N,
// equal positions, one split), so that path compiles as if they did not
// exist. SP: block-sparse, the plain forward over the tiles of the key
// blocks the block mask keeps for this query block (not with GEN).
template <typename T, int D, bool OUT_F32, bool GEN, bool SP>
__global__ __launch_bounds__(kThreads, FwdTile<D>::OCC) void fwd_mfma_kernel(FwdArgs a) {
  static_assert(!(GEN && SP), "the block-sparse form is the plain forward's");
  using L = TileLayout<D>;
  constexpr int BC = FwdTile<D>::BC;
  constexpr int KT = BC / 32;                   // 32-key sub-tiles
  constexpr int DC = D / 16;                    // 16-wide d chunks (S reduction)
  constexpr int DT = D / 32;                    // 32-wide d tiles of O^T
  constexpr int TB = L::bytes(BC);              // bytes per K or V tile

  // Two buffers each of K and V, as four separate variables: the compiler
  // can then tell a copy into one buffer from reads of the other and does
  // not make the reads wait for the copy (it would with one array of two).
  __shared__ __attribute__((aligned(1024))) unsigned char Ks0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Ks1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs1[TB];
  // Buffer of parity p; p is a compile-time constant in the main loop.
  auto kbuf = [&](int p) -> unsigned char* { return p ? Ks1 : Ks0; };
  auto vbuf = [&](int p) -> unsigned char* { return p ? Vs1 : Vs0; };
  // Block-sparse: the kept key blocks of this query block, listed.
  __shared__ unsigned short blist[SP ? kMaxMaskBlocks + 2 : 1];
  __shared__ int bwc[SP ? kWaves : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int ql = lane & 31;  // query column within the wave
  const int hh = lane >> 5;  // k-group half of the wave

  const int N = a.N;
  const int nqb = (N + kBR - 1) / kBR;
  // The key split is the outermost grid index; inside a split, blocks are
  // placed as for the whole forward.
  const int per_split = a.B * a.H * nqb;
  const int split = GEN ? blockIdx.x / per_split : 0;
  const BlockPick pk = pick_block(blockIdx.x - split * per_split, per_split, nqb, a.B * a.H, a.causal,
                                  FwdTile<D>::OCC);
  int bh = pk.bh;
  int qb = a.causal ? nqb - 1 - pk.rank : pk.rank;  // causal: last block has most work
  // Block-sparse by pieces: the workgroup's item names its row and piece.
  int piece0 = 0, slot = -1;
  const bool by_items = SP && a.sp_items != nullptr;
  if (by_items) {
    const int* it4 = a.sp_items + 4 * (size_t)blockIdx.x;
    bh = __builtin_amdgcn_readfirstlane(it4[0]);
    qb = __builtin_amdgcn_readfirstlane(it4[1]);
    piece0 = __builtin_amdgcn_readfirstlane(it4[2]);
    slot = __builtin_amdgcn_readfirstlane(it4[3]);
  }
  const int b = bh / a.H;

  const size_t head_off = (size_t)bh * N * D;          // Q and O
  const int Nk = GEN ? a.Nk : N;
  const int kvh = b * a.Hkv + (bh - b * a.H) / (a.H / a.Hkv);  // K/V head of this query head
  const size_t head_k = (size_t)kvh * Nk * D;          // K and V
  const int k_lo = GEN ? split * a.ksplit : 0;         // this split's keys: [k_lo, k_hi)
  int kv_end = GEN ? min(k_lo + a.ksplit, Nk) : N;     // keys visible at all (exclusive)
  if (a.kv_len) kv_end = min(max(a.kv_len[b], 0), kv_end);
  // causal: key j visible to query i iff j <= i + delta
  const int delta = GEN ? a.q_pos0 - a.k_pos0 : 0;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)a.q + head_off, (uint32_t)N * D * 2);
  const uint32_t kv_bytes = (uint32_t)max(kv_end, 0) * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t*)a.k + head_k, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t*)a.v + head_k, kv_bytes);

  const int q_blk0 = qb * kBR;
  const int q_blk_last = min(q_blk0 + kBR, N) - 1;
  int kv_lim = kv_end;  // keys the workgroup needs (exclusive)
  if (a.causal) kv_lim = min(kv_lim, q_blk_last + delta + 1);
  // Tiles are counted from this split's first tile jb (k_lo is a multiple of
  // the tile width); tile t holds keys [(jb + t) * BC, (jb + t + 1) * BC).
  const int jb = k_lo / BC;
  int ntiles = max((kv_lim + BC - 1) / BC - jb, 0);

  const int wq0 = q_blk0 + wave * 32;
  const int my_q = wq0 + ql;
  int w_lim = kv_end;  // keys this wave needs (exclusive)
  if (a.causal) w_lim = min(w_lim, min(wq0 + 31, N - 1) + delta + 1);
  int w_tiles = max((max(w_lim, 0) + BC - 1) / BC - jb, 0);  // tiles this wave computes

  // Block-sparse: from here on a tile count or position t counts only the
  // tiles of kept blocks, in increasing order; tile_ix(t) is the key tile.
  // A piece sees the list from its first block on, at most kSparsePiece
  // blocks of it (the entries after a piece are real blocks or the list's
  // own end copies, so a prefetch past the piece reads a tile of the head).
  int n_kept = 0;
  const unsigned short* plist = blist;
  if constexpr (SP) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const unsigned char* mrow = a.bmask + (long long)b * a.bm_sb +
                                (long long)(bh - b * a.H) * a.bm_sh + (long long)qb * nb;
    n_kept = list_mask_blocks<kThreads>(mrow, 1, 0, min(nb, (kv_lim + kMaskBlock - 1) / kMaskBlock),
                                        blist, bwc);
    if (by_items) {
      plist = blist + min(piece0, n_kept);
      n_kept = max(min(n_kept - piece0, kSparsePiece), 0);
    }
    w_tiles = mask_tiles_below(plist, n_kept, w_tiles);
    ntiles = mask_tiles_below(plist, n_kept, ntiles);
  }
  auto tile_ix = [&](int t) -> int {
    if constexpr (SP) return mask_tile(plist, t);
    else return jb + t;
  };

  u32x4 qf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qf[dc] = buf_load16(rq, (uint32_t)(my_q * D + dc * 16 + hh * 8) * 2);

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_ref = -INFINITY;  // running max of raw scores (both halves agree)
  float mref2 = 0.f;        // m_ref * scale * log2(e), 0 while m_ref is -inf
  float l_run = 0.f;        // running sum over this half's keys, against m_ref
  const float sl2 = a.scale * kLog2e;

  auto load_tile = [&](__amdgpu_buffer_rsrc_t r, unsigned char* dst, int t) {
    load_tile_lds<D, BC, kWaves>(r, dst, tile_ix(t) * BC, wave, lane);
  };

  // K fragment (A of S^T): row kt*32 + ql, chunk 2*dc + hh. The row's place
  // in its group is fixed per lane, so the swizzle folds into a per-lane
  // offset per chunk.
  int k_off[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) k_off[dc] = L::off(ql, 2 * dc + hh);
  auto compute_s = [&](const unsigned char* kb, f32x16 (&s)[KT]) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4 kf = *(const u32x4*)&kb[kt * (32 / L::RPI) * L::GB + k_off[dc]];
        s[kt] = Mfma<T>::mma32(kf, qf[dc], s[kt]);
      }
    }
  };

  // V fragment (A of O^T) via ds_read_b64_tr_b16 over the 16 keys x 32 d
  // block at rows kt*32 + c2*16, columns dt*32.
  int v_off[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) v_off[dt] = L::tr_off(lane, dt * 32);

  f32x16 s_a[KT], s_b[KT];
  if (ntiles > 0) {
    load_tile(rk, Ks0, 0);
    load_tile(rk, Ks1, 1);
    load_tile(rv, Vs0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (w_tiles > 0) compute_s(Ks0, s_a);
  }

  // One tile of the pipeline: S of tile j+1 into s_nxt, softmax and P V of
  // tile j from s_cur. FULL tiles (every row of every wave sees every key of
  // tiles j and j+1) run branch-free apart from the uniform rescale test, so
  // the S(j+1) products, the exponentials of tile j and its P V products sit
  // in one basic block and the scheduler can interleave MFMA and VALU work.
  // Other tiles (the causal diagonal, the padded or ragged end) take the
  // general path with per-wave liveness and masking.
  auto tile = [&](int j, f32x16 (&s_cur)[KT], f32x16 (&s_nxt)[KT], auto full, int par) {
    constexpr bool FULL = decltype(full)::value;
    // Every wave has finished tile j-1: the K buffer of tile j and the V
    // buffer of tile j-1 are free. Loads past the last tile read inside the
    // head, or zeros past the resource end, and are never used.
    __syncthreads();
    if (FULL || j + 2 < ntiles) load_tile(rk, kbuf(par), j + 2);
    if (FULL || j + 1 < ntiles) load_tile(rv, vbuf(par ^ 1), j + 1);
    const bool live = FULL || j < w_tiles;
    if (live) {
      if constexpr (!FULL) {
        const int t0 = tile_ix(j) * BC;
        const bool need_mask = (t0 + BC > kv_end) || (a.causal && t0 + BC - 1 > wq0 + delta);
        if (need_mask) {
          // Score r of sub-tile kt is key t0 + 4 hh + c with c = 32 kt +
          // 8 (r / 4) + r % 4 a constant, visible iff the key is at most
          // min(kv_end - 1, my_q + delta): one compare of c with a per-lane
          // bound per score.
          int lim = kv_end - 1;
          if (a.causal) lim = min(lim, my_q + delta);
          lim -= t0 + 4 * hh;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kt * 32 + 8 * (r >> 2) + (r & 3) > lim) s_cur[kt][r] = -INFINITY;
          }
        }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[kt][r]);
      }
      mx = halves_max(mx);
      if (__any(mx > m_ref)) {
        const float m_new = max_nn(m_ref, mx);
        const float alpha = (m_new == m_ref) ? 1.f : fast_exp2((m_ref - m_new) * sl2);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        m_ref = m_new;
        mref2 = (m_new == -INFINITY) ? 0.f : m_new * sl2;
      }

      // Main block of a full tile: ask the scheduler to interleave the MFMA
    // chains with the exponentials and LDS reads (iglp_opt strategy 0). At
    // d = 64 also raise this wave's issue priority while it runs, so the
    // SIMD's other waves fill the gaps rather than the other way round; at
    // d = 128 (two waves per SIMD) the raise measured 3% slower on causal
    // shapes and neutral on the others. The raise comes first: s_setprio
    // ends a scheduling region, so placed after iglp_opt it left the hint
    // an empty region and the main block the default schedule.
    if constexpr (FULL) {
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_iglp_opt(0);
    }
    if (FULL || j + 1 < w_tiles) compute_s(kbuf(par ^ 1), s_nxt);

      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s_cur[kt][r], sl2, -mref2));
          s_cur[kt][r] = p;
          lsum += p;
        }
      }
      l_run += lsum;

      // O^T += V^T P^T, 16 keys per MFMA. Rows kt*32 + c2*16 (+8) of the V
      // tile start whole groups, so they only move the group base.
      const unsigned char* vb = vbuf(par);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const u32x4 pf = {Mfma<T>::pack(s_cur[kt][8 * c2 + 0], s_cur[kt][8 * c2 + 1]),
                            Mfma<T>::pack(s_cur[kt][8 * c2 + 2], s_cur[kt][8 * c2 + 3]),
                            Mfma<T>::pack(s_cur[kt][8 * c2 + 4], s_cur[kt][8 * c2 + 5]),
                            Mfma<T>::pack(s_cur[kt][8 * c2 + 6], s_cur[kt][8 * c2 + 7])};
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const unsigned char* vp = vb + (2 * kt + c2) * L::rows16() + v_off[dt];
            const u32x2 v0 = lds_read_tr(vp);
            const u32x2 v1 = lds_read_tr(vp + L::half_step());
            const u32x4 vf = {v0.x, v0.y, v1.x, v1.y};
            oacc[dt] = Mfma<T>::mma32(vf, pf, oacc[dt]);
          }
        }
      }
      if constexpr (FULL && D == 64) __builtin_amdgcn_s_setprio(0);
    }
    // This wave's loads for the next tiles must have landed before anyone
    // passes the next barrier.
    __builtin_amdgcn_s_waitcnt(0);
  };

  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  // Tiles fully visible to every row of the workgroup, and followed by a
  // further tile, form the branch-free main loop (an even count, so the two
  // S arrays swap roles without copies).
  int n_vis = (a.causal ? min(kv_end, q_blk0 + delta + 1) : kv_end) / BC - jb;
  if constexpr (SP) n_vis = mask_tiles_below(plist, n_kept, n_vis);
  const int n_full = max(min(n_vis, ntiles - 1), 0) & ~1;
  int j = 0;
  for (; j < n_full; j += 2) {
    tile(j, s_a, s_b, Full{}, 0);
    tile(j + 1, s_b, s_a, Full{}, 1);
  }
  for (; j < ntiles; ++j) {
    tile(j, s_a, s_b, Part{}, j & 1);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) s_a[kt] = s_b[kt];
  }

  const float l_tot = halves_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (by_items && slot >= 0) {
    // the piece's fp32 O (normalised over its keys) and LSE, rows = queries
    // of the block; the merge combines a row's pieces
    const int r = wave * 32 + ql;
    float* Op = a.sp_part + ((size_t)slot * kMaskBlock + r) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + r4 * 8 + 4 * hh;
        *(f32x4*)(Op + d0) = f32x4{oacc[dt][4 * r4] * inv, oacc[dt][4 * r4 + 1] * inv,
                                   oacc[dt][4 * r4 + 2] * inv, oacc[dt][4 * r4 + 3] * inv};
      }
    }
    if (hh == 0)
      a.sp_part[(size_t)a.sp_nslots * kMaskBlock * D + (size_t)slot * kMaskBlock + r] =
          (l_tot > 0.f) ? m_ref * a.scale + fast_log2(l_tot) * kLn2 : -INFINITY;
  } else if (!OUT_F32 && !GEN) {
    // O of the wave's 32 rows through LDS (every wave is past its last
    // tile, so the K and V buffers are free) and out in whole rows.
    unsigned char* stage = wave == 0 ? Ks0 : wave == 1 ? Ks1 : wave == 2 ? Vs0 : Vs1;
    __syncthreads();
    stage_put<T, D>(stage, oacc, inv, lane);
    __syncthreads();
    stage_rows_out<D>(stage, (uint16_t*)a.o + head_off + (size_t)wq0 * D, N - wq0, lane);
    if (hh == 0 && my_q < N)
      a.lse[(size_t)bh * N + my_q] = (l_tot > 0.f) ? m_ref * a.scale + fast_log2(l_tot) * kLn2 : -INFINITY;
  } else if (my_q < N) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + r4 * 8 + 4 * hh;
        const float o0 = oacc[dt][4 * r4 + 0] * inv, o1 = oacc[dt][4 * r4 + 1] * inv;
        const float o2 = oacc[dt][4 * r4 + 2] * inv, o3 = oacc[dt][4 * r4 + 3] * inv;
        if constexpr (OUT_F32) {
          float* Og = (float*)a.o + (GEN ? split * a.o_split_stride : 0) + head_off;
          *(f32x4*)(Og + (size_t)my_q * D + d0) = f32x4{o0, o1, o2, o3};
        } else {
          uint16_t* Og = (uint16_t*)a.o + (GEN ? split * a.o_split_stride : 0) + head_off;
          *(u32x2*)(Og + (size_t)my_q * D + d0) = u32x2{Mfma<T>::pack(o0, o1), Mfma<T>::pack(o2, o3)};
        }
      }
    }
    if (hh == 0) {
      a.lse[(GEN ? split * a.lse_split_stride : 0) + (size_t)bh * N + my_q] =
          (l_tot > 0.f) ? m_ref * a.scale + fast_log2(l_tot) * kLn2 : -INFINITY;
    }
  }
}

// O and LSE of the block-sparse rows cut into pieces: the pieces' (O, LSE)
// combined by the online-softmax rule, m = max LSE_p, w_p = exp(LSE_p - m),
// O = sum w_p O_p / sum w_p, LSE = m + ln sum w_p (pieces in order). One
// wave per (row, 256 / D query rows); thread t covers 4 elements.
template <typename OutT, int D>
__global__ __launch_bounds__(kReduceThreads) void sparse_o_merge_kernel(FwdArgs a) {
  constexpr int ROWS = kReduceThreads * 4 / D;
  const int row = blockIdx.x / (kMaskBlock / ROWS);
  const int r0 = (blockIdx.x % (kMaskBlock / ROWS)) * ROWS;
  const int* c4 = a.sp_rows + 4 * (size_t)row;
  const int bh = c4[0], qb = c4[1], slot0 = c4[2], np = c4[3];
  const int e = threadIdx.x * 4;
  const int r = r0 + e / D, d0 = e % D;
  const int q = qb * kMaskBlock + r;
  if (q >= a.N) return;
  const size_t blk = (size_t)kMaskBlock * D;
  const float* lse = a.sp_part + (size_t)a.sp_nslots * blk + (size_t)slot0 * kMaskBlock + r;
  float m = -INFINITY;
  for (int i = 0; i < np; ++i) m = fmaxf(m, lse[i * kMaskBlock]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != -INFINITY) {
    const float* op = a.sp_part + (size_t)slot0 * blk + (size_t)r * D + d0;
#pragma unroll 4
    for (int i = 0; i < np; ++i) {
      const float w = fast_exp2((lse[i * kMaskBlock] - m) * kLog2e);
      const f32x4 x = *(const f32x4*)(op + i * blk);
      acc[0] += w * x[0]; acc[1] += w * x[1]; acc[2] += w * x[2]; acc[3] += w * x[3];
      den += w;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const size_t off = ((size_t)bh * a.N + q) * D + d0;
  if constexpr (std::is_same<OutT, float>::value) {
    *(f32x4*)((float*)a.o + off) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  } else {
    *(u32x2*)((uint16_t*)a.o + off) = u32x2{Mfma<OutT>::pack(acc[0] * inv, acc[1] * inv),
                                            Mfma<OutT>::pack(acc[2] * inv, acc[3] * inv)};
  }
  if (d0 == 0) a.lse[(size_t)bh * a.N + q] = den > 0.f ? m + fast_log2(den) * kLn2 : -INFINITY;
}

template <typename T, int D, bool OF, bool GEN, bool SP = false>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  if (SP && a.sp_items) {
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, OF, GEN, SP>), dim3((unsigned)a.sp_nitems), dim3(kThreads),
                       0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.sp_nrows == 0) return e;
    const dim3 g((unsigned)((long)a.sp_nrows * (kMaskBlock / (kReduceThreads * 4 / D))));
    if (OF) hipLaunchKernelGGL((sparse_o_merge_kernel<float, D>), g, dim3(kReduceThreads), 0, s, a);
    else hipLaunchKernelGGL((sparse_o_merge_kernel<T, D>), g, dim3(kReduceThreads), 0, s, a);
    return hipGetLastError();
  }
  const long nqb = (a.N + kBR - 1) / kBR;
  const long total = (long)a.B * a.H * nqb * (GEN ? a.nsplit : 1);
  hipLaunchKernelGGL((fwd_mfma_kernel<T, D, OF, GEN, SP>), dim3((unsigned)total), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

template <typename T, bool SP = false>
hipError_t launch_t(const FwdArgs& a, bool of, hipStream_t s) {
  if (a.d == 128)
    return of ? launch<T, 128, true, false, SP>(a, s) : launch<T, 128, false, false, SP>(a, s);
  return of ? launch<T, 64, true, false, SP>(a, s) : launch<T, 64, false, false, SP>(a, s);
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a, Elem in, Elem out, hipStream_t s) {
  const bool of = (out == Elem::F32);
  if (in == Elem::BF16) return launch_t<BF16>(a, of, s);
  return launch_t<F16>(a, of, s);
}

hipError_t launch_fwd_mfma_sparse(const FwdArgs& a, Elem in, Elem out, hipStream_t s) {
  const bool of = (out == Elem::F32);
  if (in == Elem::BF16) return launch_t<BF16, true>(a, of, s);
  return launch_t<F16, true>(a, of, s);
}

hipError_t launch_fwd_mfma_general(const FwdArgs& a, Elem in, hipStream_t s) {
  if (in == Elem::BF16)
    return a.d == 128 ? launch<BF16, 128, true, true>(a, s) : launch<BF16, 64, true, true>(a, s);
  return a.d == 128 ? launch<F16, 128, true, true>(a, s) : launch<F16, 64, true, true>(a, s);
}

}  // namespace fa
