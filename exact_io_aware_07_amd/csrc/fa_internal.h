// Internal declarations shared by the libfa translation units: kernel
// parameter blocks, launchers and gfx950 device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* kv_len;  // device [B] or nullptr
  int B, H, N, d;
  float scale;
  int causal;
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
};

// Launchers return hipSuccess or the launch error. Arguments are validated
// by the caller.
hipError_t launch_fwd_mfma(const FwdArgs& a, Elem in, Elem out, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
// Backward stages, launched in this order when several are asked for: the
// stand-alone D_i = rowsum(dO * O), then dQ (which also forms D_i for its
// rows and writes it to the workspace), then dK/dV (which reads D_i).
enum class BwdStage { DSUM = 1, DKDV = 2, DQ = 4, ALL = 7 };
hipError_t launch_bwd_mfma(const BwdArgs& a, Elem t, int stages, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s);

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

// Reductions across the two halves of a wave (lane l with lane l ^ 32) on
// v_permlane32_swap, a VALU op with no LDS round trip: called with (x, x) it
// returns, in lanes 0-31, (own, lane + 32) and in lanes 32-63
// (lane - 32, own), so max / sum of the pair is the two-lane result in
// every lane.
__device__ inline float halves_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
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
// position c ^ sw(r'). For D = 128 (4 rows per group) sw = 4 r'; for D = 64
// (8 rows) sw = 2 (r' / 2). With the pad, 16 lanes reading one chunk of 16
// consecutive rows, and 16 lanes reading two adjacent chunks of 4
// consecutive rows (the transposed-read pattern), fall on distinct banks.
template <int D>
struct TileLayout {
  static constexpr int RB = D * 2;       // bytes per row
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;  // rows per 1 KiB group
  static constexpr int GB = 1024 + 16;   // bytes per group incl. pad
  __device__ static constexpr int sw(int r) { return D == 128 ? 4 * r : 2 * (r >> 1); }
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
//  * Causal: work differs per block, so blocks are dispatched globally in
//    decreasing order of work (longest-processing-time first, across all
//    heads), and the hardware's round-robin over XCDs spreads that order
//    evenly. `rank` 0 is the block with the most work; the caller maps rank
//    to its own block index (the last query block, or the first key block).
struct BlockPick {
  int bh;
  int rank;
};
__device__ inline int xcd_remap(int bid, int total);
__device__ inline BlockPick pick_block(int bid, int total, int nblk, int nheads, bool causal) {
  if (causal) return BlockPick{bid % nheads, bid / nheads};
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
