// Internal declarations shared by the libfa translation units: kernel
// parameter blocks, launchers and gfx950 device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* kv_len;  // device [B] or nullptr
  int B, H, N, d;     // N: query rows per head
  float scale;
  int causal;
  // Keys and positions (the plain forward: Nk = N, both offsets 0, one split
  // of N keys, strides 0). Key j is visible to query i under the causal
  // mask when k_pos0 + j <= q_pos0 + i.
  int Nk;
  int q_pos0, k_pos0;
  int nsplit, ksplit;  // split s streams keys [s * ksplit, (s + 1) * ksplit)
  long long o_split_stride, lse_split_stride;  // elements between splits' outputs
  // K/V heads (H for plain attention): query head h of a batch uses K/V head
  // h / (H / Hkv); K and V are [B, Hkv, Nk, d].
  int Hkv;
  // Block mask of block-sparse attention (read only by that instantiation):
  // entry (b, h, i, j) at bmask[b * bm_sb + h * bm_sh + i * nb + j], nb =
  // ceil(N / kMaskBlock); nonzero keeps query block i against key block j.
  const unsigned char* bmask;
  long long bm_sb, bm_sh;
  // Block-sparse by pieces (sp_items != nullptr): workgroup i runs row item
  // sp_items[4i .. 4i+3] = (b*H + h, query block, first listed key block,
  // slot), i.e. the kept key blocks at list positions [first, first +
  // kSparsePiece) of that query block's mask row; slot < 0 writes O and
  // LSE, slot >= 0 writes the piece's fp32 O [slot][kMaskBlock][d] and LSE
  // [slot][kMaskBlock] (after all O parts) to sp_part, merged per row
  // (sp_rows[4r .. 4r+3] = (b*H + h, query block, first slot, pieces)).
  const int* sp_items;
  const int* sp_rows;
  int sp_nitems, sp_nrows, sp_nslots;
  float* sp_part;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;  // workspace: D_i = rowsum(dO * O), [B, H, N] fp32
  const int* kv_len;
  int B, H, N, d;
  float scale;
  int causal;
  // K/V heads, as in FwdArgs: K, V, dK, dV are [B, Hkv, N, d]; a K/V head's
  // gradient sums over its H / Hkv query heads.
  int Hkv;
  // gsplit > 1: each K/V head's query heads are shared among gsplit
  // workgroups per key block, which write fp32 partial dK, dV to dkv_part
  // ([2][gsplit][B, Hkv, N, d]: every dK part, then every dV part); a
  // reduction then sums the parts into dk, dv. gsplit divides H / Hkv.
  int gsplit;
  float* dkv_part;
  // Block mask, as in FwdArgs (block-sparse instantiations only).
  const unsigned char* bmask;
  long long bm_sb, bm_sh;
  // Block-sparse dK/dV by pieces (sp_items != nullptr): workgroup i runs
  // item sp_items[4i .. 4i+3] = (b*H + h, key block, first listed query
  // block, slot): the kept query blocks at list positions [first, first +
  // kSparsePiece) of that key block's column; slot < 0 writes dK, dV, slot
  // >= 0 writes fp32 partials [slot][kMaskBlock][d] (dK parts, then
  // sp_nslots dV parts) to dkv_part, which the reduction adds per column
  // (sp_cols[4c .. 4c+3] = (b*H + h, key block, first slot, pieces)).
  const int* sp_items;
  const int* sp_cols;
  int sp_nitems, sp_ncols, sp_nslots;
  // Block-sparse dQ by row pieces, as the forward's (FwdArgs::sp_*): slot
  // >= 0 writes fp32 partial dQ [slot][kMaskBlock][d] to sq_part, added per
  // row by the reduction (sq_rows).
  const int* sq_items;
  const int* sq_rows;
  int sq_nitems, sq_nrows, sq_nslots;
  float* sq_part;
  // O is fp32 (the forward's fp32 output) rather than the 16-bit input type:
  // D_i is then formed without O's 16-bit rounding.
  int o_f32;
};

// Blocks per piece of a block-sparse mask row or column.
constexpr int kSparsePiece = 8;
// Threads of the kernels that combine the pieces of a cut line: one wave.
constexpr int kReduceThreads = 64;

// Query-head split of the grouped dK/dV stage for a shape: the smallest
// divisor of H / Hkv that gives the stage at least two workgroups per
// resident slot of the chip (1 when the K/V heads alone do that).
int bwd_group_split(int B, int H, int Hkv, int N, int d);

// Launchers return hipSuccess or the launch error. Arguments are validated
// by the caller.
hipError_t launch_fwd_mfma(const FwdArgs& a, Elem in, Elem out, hipStream_t s);
// The general form (Nk, positions and key split from the arguments), fp32
// output; the plain forward above ignores those fields.
hipError_t launch_fwd_mfma_general(const FwdArgs& a, Elem in, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
// Block-sparse forward: only the tiles of the key blocks bmask keeps.
hipError_t launch_fwd_mfma_sparse(const FwdArgs& a, Elem in, Elem out, hipStream_t s);

// Block-sparse attention: masks come in blocks of kMaskBlock queries by
// kMaskBlock keys (the query block of the forward and dQ workgroups, the key
// block of the dK/dV workgroup, two 64-row tiles each). A workgroup lists
// the kept blocks of its mask row or column in LDS, so a row or column
// holds at most kMaxMaskBlocks blocks.
constexpr int kMaskBlock = 128;
constexpr int kMaxMaskBlocks = 4096;
// Backward stages, launched in this order when several are asked for: the
// stand-alone D_i = rowsum(dO * O), then dQ (which also forms D_i for its
// rows and writes it to the workspace), then dK/dV (which reads D_i).
enum class BwdStage { DSUM = 1, DKDV = 2, DQ = 4, ALL = 7 };
hipError_t launch_bwd_mfma(const BwdArgs& a, Elem t, int stages, hipStream_t s);
// Block-sparse backward stages (DQ and DKDV), skipping the blocks bmask drops.
hipError_t launch_bwd_mfma_sparse(const BwdArgs& a, Elem t, int stages, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s);

// FP8 forward with incoherent processing. Quantisation: Q and K rows
// rotated (sign flip by `signs`, unless NULL, then the unnormalised
// Walsh-Hadamard transform) and quantised to e4m3 per block (128 / 64
// rows); V per head, written transposed [B, H, d, Np] (Np = N rounded up to
// 64, zero codes past N). v_amax: [B, H, ceil(N / 64)] scratch.
struct Fp8QuantArgs {
  const void* q;
  const void* k;
  const void* v;
  const signed char* signs;
  unsigned char* q8;
  unsigned char* k8;
  unsigned char* vt8;
  float* q_scale;  // [B, H, ceil(N / 128)]
  float* k_scale;  // [B, H, ceil(N / 64)]
  float* v_scale;  // [B, H]
  float* v_amax;
  int B, H, N, d, Np;
};
struct Fp8FwdArgs {
  const unsigned char* q8;
  const unsigned char* k8;
  const unsigned char* vt8;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  void* o;
  float* lse;
  const int* kv_len;
  int B, H, N, d, Np;
  float scale;
  int causal;
  int rotated;  // scores carry the extra 1/d of the unnormalised rotation
  int o_bf16;   // 16-bit output: bf16 (1) or fp16 (0)
};
hipError_t launch_fp8_quantize(const Fp8QuantArgs& a, Elem in, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, Elem out, hipStream_t s);

// Merge of partial results (fp32 O [rows][d] and LSE [rows] per part) into
// out_o (fp32, fp16 or bf16) and out_lse. out_o / out_lse may alias part 0
// when the output is fp32.
constexpr int kMaxMergeParts = 16;
struct MergeArgs {
  const float* o[kMaxMergeParts];
  const float* lse[kMaxMergeParts];
  int nparts;
  void* out_o;
  float* out_lse;
  long long rows;
};
hipError_t launch_merge(const MergeArgs& a, int d, Elem out, hipStream_t s);

// ---------------------------------------------------------------------------
// Device helpers (gfx950).

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit element tags: the kernels move raw 16-bit words and only the MFMA
// and the fp32 <-> 16-bit conversions care which format they hold.
struct BF16 {
  static constexpr Elem kind = Elem::BF16;
};
struct F16 {
  static constexpr Elem kind = Elem::F16;
};

template <typename T>
struct Mfma;

// D(32x32, fp32) += A(32x16) * B(16x32). Lane l holds row/column l % 32 of
// its operand and the k-group l / 32; A and B map (k-group, element) to the
// reduction index the same way, so any consistent assignment of actual
// indices to those slots yields the same contraction.
template <>
struct Mfma<BF16> {
  __device__ static inline f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round-to-nearest-even pack of two fp32 into two bf16 (lo = a).
  __device__ static inline uint32_t pack(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static inline float to_f32(uint16_t x) {
    return __builtin_bit_cast(float, (uint32_t)x << 16);
  }
};

template <>
struct Mfma<F16> {
  __device__ static inline f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack(float a, float b) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 r = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static inline float to_f32(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max of two floats that are never NaN (scores, -inf for hidden keys, and
// running maxima of those) as a single v_max_f32. fmaxf first quiets each
// operand the compiler cannot prove canonical (a v_max_f32 of the value with
// itself), two extra VALU instructions per call on these operands.
__device__ inline float max_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Reductions across the two halves of a wave (lane l with lane l ^ 32) on
// v_permlane32_swap, a VALU op with no LDS round trip: called with (x, x) it
// returns, in lanes 0-31, (own, lane + 32) and in lanes 32-63
// (lane - 32, own), so max / sum of the pair is the two-lane result in
// every lane.
__device__ inline float halves_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return max_nn(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ inline float halves_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Buffer resource over [base, base + bytes): loads at or past the end read
// as zero, which is how every kernel here pads ragged tiles.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i supplies an 8-byte
// row M[i] (4 x 16-bit) and lane 4a + b receives M[a][b], M[a+4][b],
// M[a+8][b], M[a+12][b]. Pointed at a 4-row x 16-column block of a
// row-major tile (lane i at row i / 4, columns 4 * (i % 4) .. +3), every
// lane gets the 4 rows of its own column: a transposed fragment.
__device__ inline u32x2 lds_read_tr(const void* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) void*)p));
  return __builtin_bit_cast(u32x2, v);
}

// LDS layout of a [rows][D] 16-bit tile filled by direct loads: groups of
// RPI rows (1 KiB, one buffer_load ... lds per wave), each group padded by
// 16 bytes; inside a group, logical 16-byte chunk c of row r' sits at
// position c ^ sw(r'). LDS has 64 banks of 4 bytes: a 16-byte read is served
// 16 lanes per cycle, an 8-byte transposed read 32 lanes per cycle. Both
// patterns must fall on distinct banks: 16 lanes reading one chunk of 16
// consecutive rows, and 32 lanes reading four adjacent chunks (an aligned
// half-row of 4 chunks) of 4 consecutive rows. For D = 128 (4 rows per
// group, one row per 256-byte bank window) sw = 4 r'. For D = 64 (8 rows,
// two per bank window) sw is 2 x the bit-reversed r' / 2, i.e. 0 0 4 4 2 2
// 6 6: rows r' and r' + 2 then use opposite 4-chunk halves, and the four
// rows of one parity use four distinct even offsets, which the 16-byte group
// pad turns odd for the next group.
template <int D>
struct TileLayout {
  static constexpr int RB = D * 2;       // bytes per row
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;  // rows per 1 KiB group
  static constexpr int GB = 1024 + 16;   // bytes per group incl. pad
  __device__ static constexpr int sw(int r) {
    return D == 128 ? 4 * r : ((((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1));
  }
  // byte offset of logical (row, chunk) inside a tile
  __device__ static constexpr int off(int row, int chunk) {
    return (row / RPI) * GB + (row % RPI) * RB + ((chunk ^ sw(row % RPI)) << 4);
  }
  static constexpr int bytes(int rows) { return rows / RPI * GB; }
  // Byte offset, inside a tile, of the transposed-read address of `lane`
  // for the 16 x 32 block at rows [0, 16) and columns [col0, col0 + 32):
  // lanes 0-31 read rows 0-3, lanes 32-63 rows 4-7 (the second half of the
  // block, rows 8-15, is this plus half_step()); columns col0 + 16 * ((lane
  // >> 4) & 1) + 4 * (lane % 4).
  __device__ static int tr_off(int lane, int col0) {
    const int g16 = lane & 15;
    const int row = 4 * (lane >> 5) + (g16 >> 2);
    const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
    return off(row, col / 8) + (col % 8) * 2;
  }
  // offset from rows r to rows r + 8 (r a multiple of 8)
  static constexpr int half_step() { return RPI <= 8 ? (8 / RPI) * GB : 8 * RB; }
  // offset from rows r to rows r + 16 (r a multiple of 16)
  static constexpr int rows16() { return (16 / RPI) * GB; }
};

// An output tile through LDS, so that every store writes whole rows. A lane
// holds 8 bytes of a row per register group; storing those directly leaves
// each 128-byte line written in 16-byte parts by 8 separate instructions.
// Where L2 evicts lines half-written (the dK/dV stage, which streams Q and
// dO past), those lines are written back more than once. The whole-row
// stores are non-temporal: the lines go on to memory rather than staying
// dirty in L2 until the kernel ends, where writing them back delays the
// next kernel's start (by 1-3 us per kernel boundary in the GPT-2-shaped
// step). Non-temporal stores of partial lines, straight from the
// accumulators, made the kernels much slower instead.
//
// stage_put: a wave's 32 x D accumulator tile (lane l: row l % 32, elements
// dt * 32 + 8 * r4 + 4 * (l / 32) + [0, 4) in acc[dt][4 * r4 + 0..3]), times
// mul, rounded to T, into `stage` (TileLayout<D>::bytes(32) bytes).
//
// The lane index passes through an empty asm statement so that the offsets
// derived from it are computed here, after the main loop: hoisted above the
// loop they would hold registers through it.
template <typename T, int D>
__device__ inline void stage_put(unsigned char* stage, const f32x16 (&acc)[D / 32], float mul,
                                 int lane) {
  using L = TileLayout<D>;
  asm volatile("" : "+v"(lane));
  const int row = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      *(u32x2*)(stage + L::off(row, dt * 4 + r4) + 8 * hh) =
          u32x2{Mfma<T>::pack(acc[dt][4 * r4] * mul, acc[dt][4 * r4 + 1] * mul),
                Mfma<T>::pack(acc[dt][4 * r4 + 2] * mul, acc[dt][4 * r4 + 3] * mul)};
    }
  }
}

// stage_rows_out: rows [0, n) (n <= 32; none if n <= 0) of a staged tile to
// dst, row r at dst + r * D; each store writes 64 / CPR whole rows.
template <int D>
__device__ inline void stage_rows_out(const unsigned char* stage, uint16_t* dst, int n, int lane) {
  using L = TileLayout<D>;
  constexpr int RPS = 64 / L::CPR;
  asm volatile("" : "+v"(lane));
  const int cr = lane / L::CPR, cc = lane % L::CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPS; ++i) {
    const int row = i * RPS + cr;
    const u32x4 x = *(const u32x4*)(stage + L::off(row, cc));
    if (row < n) __builtin_nontemporal_store(x, (u32x4*)(dst + (size_t)row * D + cc * 8));
  }
}

// Each wave of a workgroup of `waves` fills its share of a [rows][D] tile:
// rows [row0, row0 + rows) of the tensor behind `r` go to `dst` in the
// TileLayout above. Lane l of the instruction for group G writes position
// l of that group (row l / CPR, position l % CPR), so it loads logical chunk
// (l % CPR) ^ sw(row).
template <int D, int ROWS, int WAVES>
__device__ inline void load_tile_lds(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int row0,
                                     int wave, int lane) {
  using L = TileLayout<D>;
  constexpr int GPW = ROWS / L::RPI / WAVES;
  static_assert(GPW >= 1 && ROWS % (L::RPI * WAVES) == 0, "tile too small for the workgroup");
  const int ld_row = lane / L::CPR;
  const int ld_chunk = (lane % L::CPR) ^ L::sw(ld_row);
#pragma unroll
  for (int g = 0; g < GPW; ++g) {
    const int G = wave * GPW + g;
    const int row = row0 + G * L::RPI + ld_row;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(dst + G * L::GB), 16,
        (row * D + ld_chunk * 8) * 2, 0, 0, 0);
  }
}

// Block -> (head, block-within-head) for the per-block kernels.
//  * Non-causal: every block of a head does the same work; blocks of one
//    head are kept on one XCD (xcd_remap) so its K/V stay in that L2.
//  * Causal: work differs per block. Item i = (head i % nheads, rank
//    i / nheads) has work proportional to nblk - rank, so items in index
//    order are in decreasing order of work; `rank` 0 is the block with the
//    most work and the caller maps it to its own block index (the last
//    query block, or the first key block). causal_item() chooses which item
//    each workgroup runs (see there).
struct BlockPick {
  int bh;
  int rank;
};

// Causal dispatch on MI355X. Workgroup bid runs on XCD bid % 8; the u-th
// workgroup of an XCD (u = bid / 8) goes to CU position u % 32 of that XCD
// while the kernel's first `occ` workgroups per CU are being placed (all of
// them resident at once), and later ones go wherever a slot frees. Items
// stay on the XCD of their index (item 8j + x on XCD x, so a head keeps its
// K/V in one L2 when nheads is a multiple of 8), and within an XCD the
// resident set is filled greedily, longest first: pass 0 (u < 32) takes the
// 32 longest items in order, pass 1 takes the next 32 in reverse, so the
// CU with the shortest first item gets the longest second one, and pass 2
// (occ >= 3) gives its longest item to the CU that passes 0 and 1 left least
// loaded. Workgroups from pass 3 on, and past the resident set, keep
// longest-first order. Any order is correct; this one evens out the work
// per CU when the whole grid fits on the chip at once (fewer than about
// three blocks per CU), where plain longest-first order leaves the CUs that
// drew three long blocks running alone at the end.
constexpr int kCusPerXcd = 32;
__device__ inline int causal_item(int bid, int total, int nblk, int nheads, int occ) {
  const int x = bid & 7;
  const int u = bid >> 3;
  if (u < kCusPerXcd || u >= kCusPerXcd * min(occ, 3)) return bid;
  const int n = (total - x + 7) >> 3;  // workgroups (and items) of this XCD
  const int rho = u / kCusPerXcd;
  const int c = u % kCusPerXcd;
  const int m = min(n - rho * kCusPerXcd, kCusPerXcd);  // positions used by this pass
  if (rho == 1) return 8 * (kCusPerXcd + (m - 1 - c)) + x;
  // Pass 2: load of position p after passes 0 and 1 is w(p) + w(63 - p)
  // (pass 1 is full, since pass 2 exists); rank this position among the
  // pass's m positions by that load (ties: lower position first). One lane
  // per position, then a ballot.
  auto w = [&](int j) { return nblk - (8 * j + x) / nheads; };
  const int p = threadIdx.x & (kCusPerXcd - 1);
  const int lane = threadIdx.x & 63;
  const int l_me = w(c) + w(2 * kCusPerXcd - 1 - c);
  const int l_p = w(p) + w(2 * kCusPerXcd - 1 - p);
  const bool before = lane < kCusPerXcd && p < m && (l_p < l_me || (l_p == l_me && p < c));
  const int r = __popcll(__ballot(before));
  return 8 * (2 * kCusPerXcd + r) + x;
}

// The kept blocks among [lo, hi) of one block-mask row (stride 1) or column
// (stride = blocks per row) starting at m, listed in increasing order in
// list by the whole workgroup of NT threads (a ballot per wave, the waves'
// counts through LDS). Two copies of the last kept block (or of block 0)
// follow the list, so that a prefetch one or two tiles past its end reads a
// tile of the head. Returns the count, the same in every thread.
template <int NT>
__device__ inline int list_mask_blocks(const unsigned char* __restrict__ m, long long stride, int lo,
                                       int hi, unsigned short* list, int* wcount) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  int base = 0;
  for (int c0 = lo; c0 < hi; c0 += NT) {
    const int blk = c0 + tid;
    const bool on = blk < hi && m[(long long)blk * stride] != 0;
    const unsigned long long bal = __ballot(on);
    if (lane == 0) wcount[wave] = __popcll(bal);
    __syncthreads();
    int off = base, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      // the same LDS word in every lane: uniform, so kept in an SGPR
      const int c = __builtin_amdgcn_readfirstlane(wcount[w]);
      off += (w < wave) ? c : 0;
      tot += c;
    }
    if (on) list[off + __popcll(bal & ((1ull << lane) - 1))] = (unsigned short)blk;
    base += tot;
    // every wave has read wcount before the next chunk overwrites it
    __syncthreads();
  }
  if (tid < 2) list[base + tid] = base > 0 ? list[base - 1] : (unsigned short)0;
  __syncthreads();
  return base;
}

// Tiles of a listed sequence (block b holds tiles 2b and 2b + 1) whose
// index is below lim: the sequence position of the first tile at or past
// lim. The list is increasing, so a binary search. n and lim are the same
// in every lane, so every lane reads the same entries: the entries pass
// through readfirstlane, and the search runs on scalar registers and
// branches (read from LDS, they would look divergent to the compiler, and
// so would every loop bound derived from the result).
__device__ inline int mask_tiles_below(const unsigned short* list, int n, int lim) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (2 * __builtin_amdgcn_readfirstlane((int)list[mid]) < lim) lo = mid + 1;
    else hi = mid;
  }
  const int last = lo > 0 ? __builtin_amdgcn_readfirstlane((int)list[lo - 1]) : 0;
  return 2 * lo - ((lo > 0 && 2 * last + 1 >= lim) ? 1 : 0);
}

// Tile index of sequence position t (wave-uniform, in an SGPR).
__device__ inline int mask_tile(const unsigned short* list, int t) {
  return __builtin_amdgcn_readfirstlane(2 * (int)list[t >> 1] + (t & 1));
}

__device__ inline int xcd_remap(int bid, int total);
// occ: workgroups of this kernel that fit on one CU at once.
__device__ inline BlockPick pick_block(int bid, int total, int nblk, int nheads, bool causal,
                                       int occ) {
  if (causal) {
    const int i = causal_item(bid, total, nblk, nheads, occ);
    return BlockPick{i % nheads, i / nheads};
  }
  const int logical = xcd_remap(bid, total);
  return BlockPick{logical / nblk, logical % nblk};
}

// Block index remap so that consecutive logical blocks run on the same XCD.
// Workgroups are dealt round-robin to the 8 XCDs; logical block
// x * per + i is placed on physical slot i * 8 + x. Blocks past the largest
// multiple of 8 keep their index.
__device__ inline int xcd_remap(int bid, int total) {
  const int nxcd = 8;
  const int per = total / nxcd;
  if (bid >= per * nxcd) return bid;
  return (bid % nxcd) * per + bid / nxcd;
}

}  // namespace fa
