// Sparse attention of the retrieval heads over given index sets.
//
// "Full Attention Strikes Back" (RTPurbo) section 3.2, eq. (5): retrieval
// heads attend over their Top-P set, O = sum_{n in S} softmax(q . k_n /
// sqrt(d_h)) v_n with the post-RoPE query and keys.
//
// An HBM-bound gather of bf16 rows: 16 lanes cover one 256-byte row (16 bytes
// each, coalesced); a wave holds 4 rows per step; split-K workgroups write
// softmax states that the last workgroup of each query combines.
#include "block_util.h"

namespace rtp {

namespace {

constexpr float kScale = 0.08838834764831845f;   // 1 / sqrt(128)

struct SpShared {
  float q[kD];
  int list[1024];
  int flag;
  Partial extra;
  AttnShared at;
  double2 rope[kD / 2];
  CombineShared cb;
};

// Sparse attention over a given index list: one workgroup per (query, chunk).
__global__ __launch_bounds__(kWG) void sparse_attn_kernel(Geo g, const rtp_bf16 *__restrict__ q_pre,
                                                          const rtp_bf16 *__restrict__ kc,
                                                          const rtp_bf16 *__restrict__ vc,
                                                          const int32_t *__restrict__ idx,
                                                          const int32_t *__restrict__ count, long long cap,
                                                          float *__restrict__ out) {
  __shared__ SpShared sm;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / kSpChunks, ch = blockIdx.x % kSpChunks;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const int hq = g.rhead[r], kvg = hq / g.G;
  const long long m = g.N - g.nq + i;
  rope_table(m, g.theta, sm.rope);
  rotate_query(q_pre + (((size_t)b * g.Hq + hq) * g.nq + i) * kD, sm.rope, kScale, sm.q);
  long long cnt = count[unit];
  if (cnt > cap) cnt = cap;
  if (cnt < 0) cnt = 0;
  const long long per = (cnt + kSpChunks - 1) / kSpChunks;
  const long long a0 = (long long)ch * per;
  const long long a1 = a0 + per < cnt ? a0 + per : cnt;
  const size_t cbase = kv_group_base(g, b, kvg) * kD;
  // running state of this chunk: thread d < 128 holds channel d
  float run_m = -INFINITY, run_l = 0.f, run_o = 0.f;
  for (long long s0 = a0; s0 < a1; s0 += 1024) {
    const int n = (int)(a1 - s0 < 1024 ? a1 - s0 : 1024);
    __syncthreads();
    for (int x = tid; x < n; x += kWG) sm.list[x] = idx[(size_t)unit * cap + s0 + x];
    __syncthreads();
    attend_rows(sm.q, sm.list, n, g.N, kc + cbase, vc + cbase, &sm.extra, &sm.at);
    if (tid < kD) merge_state(run_m, run_l, &run_o, sm.extra.m, sm.extra.l, &sm.extra.o[tid], 1);
  }
  Partial *dst = g.part + (size_t)unit * kSpChunks + ch;
  if (tid < kD) {
    st_coherent(&dst->o[tid], run_o);
    if (tid == 0) {
      st_coherent(&dst->m, run_m);
      st_coherent(&dst->l, run_l);
    }
  }
  if (!arrive_last(g.ctr_fin + (size_t)unit * g.cstride, (uint32_t)kSpChunks, &sm.flag)) return;
  combine_partials(g.part + (size_t)unit * kSpChunks, kSpChunks, out + (((size_t)b * g.Hq + hq) * g.nq + i) * kD,
                   &sm.cb);
}

}  // namespace

int launch_sparse_attn(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *k, const rtp_bf16 *v, const int32_t *idx,
                       const int32_t *count, long long cap, float *out, hipStream_t s) {
  if (g.units == 0) return RTP_OK;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)((long long)g.units * kSpChunks)), dim3(kWG), 0, s, g, q_pre,
                     k, v, idx, count, cap, out);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

}  // namespace rtp
