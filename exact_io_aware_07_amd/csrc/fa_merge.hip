// (O, LSE) merge of partial attention results over disjoint key sets.
//
// A partial result is attention over one part of the keys: O_p normalised
// over that part and LSE_p, the log of its softmax denominator (LSE = -inf
// when the part has no visible key for the row). The online-softmax
// recurrence (marketmaker.cc article "Flash attention and the
// sequence-length question", section "在线softmax递归") combines finished
// parts exactly as it combines tiles: with m = max_p LSE_p and
// w_p = exp(LSE_p - m),
//     O = sum_p w_p O_p / sum_p w_p,   LSE = m + ln sum_p w_p.
// This is also the step that merges the blocks a device receives in ring
// attention (Ultralytics glossary, section "Flash Attention e termini
// correlati"). A row empty in every part gets O = 0, LSE = -inf.
//
// One row per D/4 lanes, each lane owning 4 consecutive elements; a row's
// lanes are in one wave, so every read of a row precedes its writes and the
// output may alias part 0 (fp32 output).
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kMergeThreads = 256;

template <int D, typename OutT>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;                 // lanes per row
  constexpr int RPB = kMergeThreads / LPR;   // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = (threadIdx.x % LPR) * 4;
  if (row >= a.rows) return;

  float m = -INFINITY;
  for (int p = 0; p < a.nparts; ++p) m = fmaxf(m, a.lse[p][row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != -INFINITY) {
    for (int p = 0; p < a.nparts; ++p) {
      const float l = a.lse[p][row];
      if (l == -INFINITY) continue;
      const float w = fast_exp2((l - m) * kLog2e);
      const f32x4 x = *(const f32x4*)(a.o[p] + row * D + c);
      acc += w * x;
      den += w;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const f32x4 out = acc * inv;
  if constexpr (std::is_same<OutT, float>::value) {
    *(f32x4*)((float*)a.out_o + row * D + c) = out;
  } else {
    *(u32x2*)((uint16_t*)a.out_o + row * D + c) =
        u32x2{Mfma<OutT>::pack(out[0], out[1]), Mfma<OutT>::pack(out[2], out[3])};
  }
  if (c == 0) a.out_lse[row] = den > 0.f ? m + fast_log2(den) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(const MergeArgs& a, Elem out, hipStream_t s) {
  constexpr int RPB = kMergeThreads / (D / 4);
  const long long blocks = (a.rows + RPB - 1) / RPB;
  if (out == Elem::F32)
    hipLaunchKernelGGL((merge_kernel<D, float>), dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, a);
  else if (out == Elem::BF16)
    hipLaunchKernelGGL((merge_kernel<D, BF16>), dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<D, F16>), dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int d, Elem out, hipStream_t s) {
  return d == 128 ? launch_d<128>(a, out, s) : launch_d<64>(a, out, s);
}

}  // namespace fa
