// RoPE stage: Eq. 6 of "When Precision Meets Position" (arXiv 2411.13476), as
// given on the paper-graph architecture page, section 3.4: block p of the
// block-diagonal rotation R_{i,theta} turns the adjacent pair (2p, 2p+1) by
// i * theta_p, theta_p = base^(-2p/d).  Section 3.4, "Implementation detail:
// where precision matters": the rotation runs in float32 outside the
// attention kernel and the rotated vectors are rounded to bfloat16.
//
// Precision of this implementation: the angle pos * theta_p is formed and
// range-reduced in float64 (a float32 product would already be off by up to
// ~4e-3 rad at position 65535), cos and sin are rounded to float32, the pair
// is rotated with float32 fused multiply-adds and the result is rounded to
// bfloat16 to nearest even.
//
// The cos/sin table is indexed by position ID (not by token): positions are
// row-local and below S, and every head and token with that ID shares it.
#include "aa_internal.h"

namespace aa {

// table[(pos * (D/2) + p) * 2 + {0,1}] = {cos, sin}(pos * theta_p).  The
// first kernel of a call: it also clears the call's device status word and
// the counters the plan build adds to (either may be null).
__global__ void k_rope_table(int S, int half, RopeTheta th, float* __restrict__ table,
                             int32_t* __restrict__ status, int32_t* __restrict__ zero, int n_zero) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0 && status) status[0] = kStatusOk;
  if (zero && i < n_zero) zero[i] = 0;
  if (i >= (long long)S * half) return;
  const int p = (int)(i % half);
  const long long pos = i / half;
  const double ang = (double)pos * th.t[p];
  double s, c;
  sincos(ang, &s, &c);
  table[2 * i] = (float)c;
  table[2 * i + 1] = (float)s;
}

// One thread per 8 consecutive features (4 pairs) of one (token, head).
// Positions are clamped into the table's npos rows.  With src, output token
// p takes its input from token src[p] (a gather fused into the rotation).
__global__ void k_rope_apply(const bf16* __restrict__ x, const int32_t* __restrict__ src,
                             const int32_t* __restrict__ pos, const float* __restrict__ table,
                             long long n_chunks, int npos, int H, int D, bf16* __restrict__ y) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_chunks) return;
  const int chunks_per_tok = H * D / 8;
  const long long tok = i / chunks_per_tok;
  const int within = (int)(i % chunks_per_tok);
  const int d0 = (within % (D / 8)) * 8;
  const int p = min(max(pos[tok], 0), npos - 1);  // table rows exist for 0 <= pos < npos
  const long long in = src ? (long long)src[tok] * chunks_per_tok + within : i;
  const bf16x8 xv = *(const bf16x8*)(x + in * 8);
  *(bf16x8*)(y + i * 8) = rope_rotate8(xv, table + ((size_t)p * (D / 2) + d0 / 2) * 2);
}

hipError_t launch_rope_table(int S, int D, const RopeTheta& th, float* table, int32_t* status,
                             int32_t* zero, int n_zero, hipStream_t st) {
  long long n = (long long)S * (D / 2);
  if (zero && n_zero > n) n = n_zero;
  const int threads = 256;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + threads - 1) / threads)), dim3(threads), 0,
                     st, S, D / 2, th, table, status, zero, n_zero);
  return hipGetLastError();
}

hipError_t launch_rope_apply(const bf16* x, const int32_t* src, const int32_t* pos,
                             const float* table, int npos, int B, int S, int H, int D, bf16* x_rot,
                             hipStream_t st) {
  const long long n = (long long)B * S * H * D / 8;
  const int threads = 256;
  hipLaunchKernelGGL(k_rope_apply, dim3((unsigned)((n + threads - 1) / threads)), dim3(threads), 0,
                     st, x, src, pos, table, n, npos, H, D, x_rot);
  return hipGetLastError();
}

}  // namespace aa
