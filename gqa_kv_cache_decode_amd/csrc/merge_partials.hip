// Separate merge of shared segments, for shapes whose segments are split
// over many workgroups (few long sequences, large head groups). Merging such
// a segment inside the decode kernel falls to the one workgroup that arrives
// last and reads every partial slot alone; here one workgroup per (segment,
// query head) merges in parallel right after the decode launch.
//
// The combination is the one of gqa_internal.hpp: with partial states
// (m_k, l_k, o_k) of one head's pieces (base-2 running max, sum of weights,
// unnormalised output), M = max_k m_k and
//   out = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k.
//
// Workgroup (segment, head): the 256 threads are split into K = 256 / (d/4)
// groups; group r takes slots r, r + K, ... and thread c of a group one
// 16-byte column of the head's output row; the groups are combined in LDS.
#include "gqa_internal.hpp"

namespace gqa {
namespace {

template <typename TOut>
__global__ __launch_bounds__(kThreads) void merge_partials_kernel(DecodeParams p) {
  __shared__ float sm_max[kThreads];
  __shared__ __attribute__((aligned(16))) float sm_acc[kThreads * 4];
  __shared__ float sm_den[kThreads];

  const int gblk = p.gblk;
  const int seg = blockIdx.x / gblk;
  const int hh = blockIdx.x - seg * gblk;
  const int s = seg / p.ngroups;
  const int grp = seg - s * p.ngroups;
  const int j = grp / p.nhb;
  const int hb = grp - j * p.nhb;
  const int nh = min(gblk, p.G * p.n_tok - hb * gblk);  // virtual heads of a multi-token call
  if (hh >= nh) return;
  const int2 info = p.seg_info[seg];
  if (info.y < 0) return;  // written out by the decode kernel (or empty)
  const int p0 = info.x, n = info.y - info.x + 1;

  const int d = p.d;
  const int d4 = d / 4;
  const int groups = kThreads / d4;
  const int tid = threadIdx.x;
  const int r = tid / d4, c = tid - r * d4;
  const __amdgpu_buffer_rsrc_t rs = slots_rsrc(p);
  const int slot_bytes = p.slot_floats * int(sizeof(float));
  const int m_off = (gblk * d + hh) * int(sizeof(float));
  const int l_off = (gblk * d + gblk + hh) * int(sizeof(float));
  const int o_off = (hh * d + 4 * c) * int(sizeof(float));
  auto slot_base = [&](int k) { return ((p0 + k) * 2 + (k == 0 ? 1 : 0)) * slot_bytes; };

  // Each group keeps its own running max over the slots it reads, four slots
  // in flight at a time, so the slots are read in one pass; the groups are
  // combined by their maxima at the end.
  f32x4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f;
  float mrun = kNegInf;
  auto absorb = [&](float mk, float lk, f32x4v ok) {
    const float mn = fmaxf(mrun, mk);
    const float sub = (mn == kNegInf) ? 0.0f : mn;
    const float a = fast_exp2(mrun - sub), wgt = fast_exp2(mk - sub);
    den = fmaf(wgt, lk, den * a);
    acc = acc * a + wgt * ok;
    mrun = mn;
  };
  int k = r;
  for (; k + 3 * groups < n; k += 4 * groups) {
    float mk[4], lk[4];
    f32x4v ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int base = slot_base(k + u * groups);
      mk[u] = coherent_load1(rs, base + m_off);
      lk[u] = coherent_load1(rs, base + l_off);
      ok[u] = coherent_load4(rs, base + o_off);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) absorb(mk[u], lk[u], ok[u]);
  }
  for (; k < n; k += groups) {
    const int base = slot_base(k);
    absorb(coherent_load1(rs, base + m_off), coherent_load1(rs, base + l_off), coherent_load4(rs, base + o_off));
  }
  *reinterpret_cast<f32x4v*>(&sm_acc[4 * tid]) = acc;
  sm_den[tid] = den;
  if (c == 0) sm_max[r] = mrun;
  __syncthreads();
  if (tid < d4) {
    float M = sm_max[0];
    for (int rr = 1; rr < groups; ++rr) M = fmaxf(M, sm_max[rr]);
    const float sub = (M == kNegInf) ? 0.0f : M;
    f32x4v o = {0.0f, 0.0f, 0.0f, 0.0f};
    float dsum = 0.0f;
    for (int rr = 0; rr < groups; ++rr) {
      const float wgt = fast_exp2(sm_max[rr] - sub);
      o += wgt * *reinterpret_cast<const f32x4v*>(&sm_acc[4 * (rr * d4 + tid)]);
      dsum = fmaf(wgt, sm_den[rr * d4 + tid], dsum);
    }
    const float inv = dsum > 0.0f ? 1.0f / dsum : 0.0f;
    TOut* out = static_cast<TOut*>(p.out);
    const size_t o0 = head_row(p.n_tok, p.h, p.G, s, j * p.G * p.n_tok + hb * gblk + hh) * d + 4 * tid;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(out, o0 + e, o[e] * inv);
  }
}

}  // namespace

hipError_t launch_merge_partials(const DecodeParams& p, int dtype, hipStream_t stream) {
  const dim3 grid(unsigned(p.b) * unsigned(p.ngroups) * unsigned(p.gblk));
  if (dtype == 0)
    hipLaunchKernelGGL(merge_partials_kernel<float>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_partials_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
