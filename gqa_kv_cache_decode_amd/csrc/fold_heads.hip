// Mean-fold of KV heads: a cache (or a key/value projection) with g_src KV
// heads becomes one with g_dst heads, each contiguous group of F = g_src /
// g_dst heads replaced by its average ("TF2 GQA" lesson, on turning a trained
// multi-head model into a grouped one: the key/value heads of a group are
// averaged; the lesson's lab folds contiguous groups by their mean).
//
//   dst[s][j][t][c] = (sum_{f<F} src[s][j*F + f][t][c]) / F      t < rows_s
//
// The sum runs in head order in double precision and the mean is rounded
// once to the element type, so the result does not depend on how the work
// is cut. Reading F rows per written row, the kernel is bound by HBM: each
// thread owns 8 consecutive elements of one (sequence, folded head) run, and
// a workgroup 2048 consecutive elements, so the loads of a wave cover
// contiguous 1 KiB (bf16) pieces of each source head.
#include "gqa_internal.hpp"

namespace gqa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFoldThreads = 256;
constexpr int kFoldElems = 8;  // elements per thread

// A double rounded once to bf16, nearest even. The double is first rounded
// to fp32 with round-to-odd (truncate, then set the last bit if anything was
// cut); fp32 keeps 16 bits more than bf16, so rounding that value to bf16 to
// nearest even gives the same result as rounding the double directly (the
// classic round-to-odd argument: at least two extra bits make the second
// rounding innocuous). A NaN becomes the canonical quiet NaN 0x7fc0.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  if (x != x) return uint16_t(0x7fc0u);
  float f = static_cast<float>(x);  // nearest even
  uint32_t u = __float_as_uint(f);
  const double back = static_cast<double>(f);
  if (back != x) {
    if (fabs(back) > fabs(x)) u -= 1u;  // step the magnitude back toward zero: truncation
    u |= 1u;                            // sticky bit
  }
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <typename T>
__global__ __launch_bounds__(kFoldThreads) void fold_heads_kernel(FoldParams p) {
  const int s = blockIdx.z;
  const int j = blockIdx.y;
  const int rows = p.lens ? min(max(p.lens[s], 0), p.max_rows) : p.max_rows;
  const size_t e0 = (size_t(blockIdx.x) * kFoldThreads + threadIdx.x) * kFoldElems;
  if (e0 >= size_t(rows) * size_t(p.d)) return;  // d % 8 == 0: the 8 elements share a row
  const int F = p.g_src / p.g_dst;
  const size_t run_src = size_t(p.cap_src) * size_t(p.d);
  const T* src = static_cast<const T*>(p.src) + (size_t(s) * p.g_src + size_t(j) * F) * run_src + e0;

  double acc[kFoldElems];
#pragma unroll
  for (int e = 0; e < kFoldElems; ++e) acc[e] = 0.0;
  constexpr int kVecs = kFoldElems * int(sizeof(T)) / 16;  // 16-byte loads per head
#pragma unroll 4
  for (int f = 0; f < F; ++f) {
    const u32x4* ptr = reinterpret_cast<const u32x4*>(src + size_t(f) * run_src);
    u32x4 v[kVecs];
#pragma unroll
    for (int k = 0; k < kVecs; ++k) v[k] = __builtin_nontemporal_load(ptr + k);
#pragma unroll
    for (int k = 0; k < kVecs; ++k)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (sizeof(T) == 2) {
          acc[8 * k + 2 * w] += static_cast<double>(__uint_as_float(v[k][w] << 16));
          acc[8 * k + 2 * w + 1] += static_cast<double>(__uint_as_float(v[k][w] & 0xffff0000u));
        } else {
          acc[4 * k + w] += static_cast<double>(__uint_as_float(v[k][w]));
        }
      }
  }

  const size_t run_dst = size_t(p.cap_dst) * size_t(p.d);
  T* dst = static_cast<T*>(p.dst) + (size_t(s) * p.g_dst + j) * run_dst + e0;
  const double fd = static_cast<double>(F);
  if constexpr (sizeof(T) == 2) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      o[w] = uint32_t(f64_to_bf16(acc[2 * w] / fd)) | (uint32_t(f64_to_bf16(acc[2 * w + 1] / fd)) << 16);
    *reinterpret_cast<u32x4*>(dst) = o;
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = __float_as_uint(static_cast<float>(acc[4 * k + w] / fd));
      reinterpret_cast<u32x4*>(dst)[k] = o;
    }
  }
}

}  // namespace

hipError_t launch_fold(const FoldParams& p, int b, int dtype, hipStream_t stream) {
  const size_t elems = size_t(p.max_rows) * size_t(p.d);
  const size_t chunks = (elems + size_t(kFoldThreads) * kFoldElems - 1) / (size_t(kFoldThreads) * kFoldElems);
  const dim3 grid(unsigned(chunks), unsigned(p.g_dst), unsigned(b));
  if (dtype == 0) hipLaunchKernelGGL(fold_heads_kernel<float>, grid, dim3(kFoldThreads), 0, stream, p);
  else hipLaunchKernelGGL(fold_heads_kernel<uint16_t>, grid, dim3(kFoldThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
