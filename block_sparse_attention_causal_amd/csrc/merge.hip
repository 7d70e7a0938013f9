// a5: log-sum-exp merge of the attention parts of every row.
//
// Kimi发布MoBA突破性实现无限上下文, "PyTorch实现关键要点": the self-block part and
// the selected-block parts are combined with an online softmax. Each part p is
// a normalised output o_p with its log-sum-exp lse_p over a disjoint key set,
// so the exact softmax over the union is
//   out = sum_p exp(lse_p - m) o_p / sum_p exp(lse_p - m),  m = max_p lse_p,
//   lse = m + log(sum_p exp(lse_p - m)).
// A row of query block i has min(topk-1, i) selected parts (slots 0..n-1).
#include "moba_plan.h"

namespace moba {

template <typename T, int D>
__global__ void __launch_bounds__(256) k_merge(const int32_t* __restrict__ cu, int nseq, int hq,
                                               int block, int ks, int64_t rows,
                                               const typename PartType<T>::type* __restrict__ o_self,
                                               const float* __restrict__ lse_self,
                                               const typename PartType<T>::type* __restrict__ o_sel,
                                               const float* __restrict__ lse_sel,
                                               T* __restrict__ out, float* __restrict__ lse_out) {
  typedef typename PartType<T>::type P;
  constexpr int TPR = D / 8;            // threads per row, 8 values each
  constexpr int RPW = 256 / TPR;        // rows per workgroup
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c = threadIdx.x % TPR;
  const int64_t tok = row / hq;
  const int n = seq_of_token(cu, nseq, tok);
  const int i = (int)((tok - cu[n]) / block);
  const int nsel = min(ks, i);
  const float ls = lse_self[row];
  float m = ls;
  for (int sl = 0; sl < nsel; ++sl) m = fmaxf(m, lse_sel[row * ks + sl]);
  float wgt = fast_exp2((ls - m) * kLog2e);
  float den = wgt;
  float acc[8];
  {
    const P* src = o_self + row * D + 8 * c;
    float x[8];
    load8_part(src, x);
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = x[b] * wgt;
  }
  for (int sl = 0; sl < nsel; ++sl) {
    const int64_t e = row * ks + sl;
    wgt = fast_exp2((lse_sel[e] - m) * kLog2e);
    den += wgt;
    float x[8];
    load8_part(o_sel + e * D + 8 * c, x);
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] += x[b] * wgt;
  }
  const float inv = 1.f / den;
  typedef T vec4_t __attribute__((ext_vector_type(4)));
  vec4_t r0, r1;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    r0[b] = from_f32<T>(acc[b] * inv);
    r1[b] = from_f32<T>(acc[4 + b] * inv);
  }
  T* dst = out + row * D + 8 * c;
  __builtin_nontemporal_store(r0, reinterpret_cast<vec4_t*>(dst));
  __builtin_nontemporal_store(r1, reinterpret_cast<vec4_t*>(dst + 4));
  if (lse_out && c == 0) lse_out[row] = m + fast_log2(den) * kLn2;
}

hipError_t launch_merge(const Plan& p, const int32_t* cu_dev, const Work& w, void* out,
                        float* lse_out, hipStream_t s) {
  const int64_t rows = p.T * p.hq;
  if (p.ks == 0 || rows == 0) return hipSuccess;
  const int rpw = 256 / (p.d / 8);
  dim3 grid((unsigned)((rows + rpw - 1) / rpw)), blk(256);
  if (p.dtype == MOBA_DTYPE_BF16) {
    if (p.d == 128)
      hipLaunchKernelGGL((k_merge<bf16, 128>), grid, blk, 0, s, cu_dev, p.nseq, p.hq, p.block,
                         p.ks, rows, (const f16*)w.o_self, w.lse_self, (const f16*)w.o_sel, w.lse_sel,
                         (bf16*)out, lse_out);
    else
      hipLaunchKernelGGL((k_merge<bf16, 64>), grid, blk, 0, s, cu_dev, p.nseq, p.hq, p.block,
                         p.ks, rows, (const f16*)w.o_self, w.lse_self, (const f16*)w.o_sel, w.lse_sel,
                         (bf16*)out, lse_out);
  } else {
    if (p.d == 128)
      hipLaunchKernelGGL((k_merge<float, 128>), grid, blk, 0, s, cu_dev, p.nseq, p.hq, p.block,
                         p.ks, rows, (const float*)w.o_self, w.lse_self, (const float*)w.o_sel,
                         w.lse_sel, (float*)out, lse_out);
    else
      hipLaunchKernelGGL((k_merge<float, 64>), grid, blk, 0, s, cu_dev, p.nseq, p.hq, p.block,
                         p.ks, rows, (const float*)w.o_self, w.lse_self, (const float*)w.o_sel,
                         w.lse_sel, (float*)out, lse_out);
  }
  return hipGetLastError();
}

}  // namespace moba
