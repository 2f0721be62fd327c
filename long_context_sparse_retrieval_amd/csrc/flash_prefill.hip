// Prefill attention on the matrix cores: causal attention of nq queries per
// head, dense for retrieval heads and sliding window plus sinks for local
// heads, or dense for every head (the comparator).
//
// "Full Attention Strikes Back" (RTPurbo) section 3.2: during prefill the
// retrieval heads keep the full KV cache (dense causal attention) while the
// local heads attend to a sliding window with attention sinks; the attention
// itself is eq. (5)'s softmax(q . k / sqrt(d_h)) V.  The DeepRead summary's
// "Key Results" compare this prefill against dense attention for every head.
//
// Design for gfx950.  A workgroup takes 16 consecutive queries of up to four
// q heads of one KV group and one mode (one wave per head), so every K/V block
// staged in LDS serves four heads.  Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_16x16x32_bf16 (K = 32 per instruction, twice
// the rate of the K = 16 form on gfx950): the keys are the A operand and the
// queries the B operand, so each lane ends up with four keys of one query per
// 16-key subtile; two subtiles fill the eight slots of P's A operand for a
// K = 32 step of O += P V, and V, staged transposed, is read in the same slot
// order.  The rotated query (fp64 angles) and the softmax weights P are
// each split into two bf16 halves, x = hi + lo, so both products carry
// fp32-level precision (bf16 P alone misses the 2e-3 output bar when a few
// keys dominate).  The softmax runs online in base 2 (log2(e) / sqrt(d)
// folded into the query); a query's running maximum and sum sit in the four
// lanes that hold it.
#include <string.h>

#include "block_util.h"

namespace rtp {

namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFq = 16;                 // queries per wave (the matrix-core N dimension)
constexpr int kFk = 64;                 // keys per staged block
constexpr int kKPad = kD + 8;           // padded key row in LDS (elements)
constexpr int kVPad = kFk + 4;          // padded row of transposed values (elements)
constexpr double kQScale = 1.4426950408889634 / 11.313708498984761;   // log2(e) / sqrt(128)
constexpr float kLazy = 8.f;            // headroom of the running maximum (base 2)
constexpr int kBufs = 1;               // LDS buffers per K/V block (1: a second barrier per block)

struct FlashShared {
  rtp_bf16 k[kBufs][kFk][kKPad];        // keys of a block, row-major
  rtp_bf16 vt[kBufs][kD][kVPad];        // values of a block, transposed
};

// fp32 -> bf16, nearest even (one v_cvt_pk_bf16_f32 per pair on gfx950)
__device__ __forceinline__ short bf16_rne(float x) { return __builtin_bit_cast(short, (__bf16)x); }

__device__ __forceinline__ float bf16_f(short b) { return __uint_as_float((uint32_t)(uint16_t)b << 16); }

__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(3, 8))) void flash_prefill_kernel(Geo g, FlashQuads fq, const rtp_bf16 *__restrict__ q_pre,
                                                            const rtp_bf16 *__restrict__ kc,
                                                            const rtp_bf16 *__restrict__ vc, float *__restrict__ out,
                                                            int ntiles) {
  __shared__ FlashShared sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups x and x + 8 share an XCD.  Each (quad, sequence) deals its
  // query tiles to the eight XCDs in turn, so a dense quad's work spreads over
  // the whole chip (dealing strips of consecutive tiles to one XCD was
  // measured slower); the longest tiles come first.
  const int inner = fq.n * g.B;
  const int y = (int)(blockIdx.x >> 3);
  const int rank = (y / inner) * 8 + (int)(blockIdx.x & 7);
  if (rank >= ntiles) return;                                  // padding to whole XCD rounds
  const int tile = ntiles - 1 - rank;
  const int rest = y % inner;
  const int quad = rest % fq.n, b = rest / fq.n;
  const bool has_head = wv < fq.nh[quad];                     // false: this wave only helps staging
  const int h0 = fq.head[4 * quad];
  const int h = has_head ? fq.head[4 * quad + wv] : h0;
  const bool dense = fq.dense[quad] != 0;
  const int kvg = h0 / g.G;
  const int i0 = tile * kFq;
  const int nqt = g.nq - i0 < kFq ? g.nq - i0 : kFq;
  const long long m0 = g.N - g.nq + i0, m_hi = m0 + nqt - 1;
  const int qn = lane & 15, grp = lane >> 4;
  const size_t cbase = kv_group_base(g, b, kvg);

  // this lane's query (qn) as the B operand of the K = 32 products: dims
  // 32 c + 8 grp .. + 7, split hi + lo
  bf16x8_t qh[kD / 32], ql[kD / 32];
  {
    const int qi = i0 + (qn < nqt ? qn : nqt - 1);
    const long long mq = g.N - g.nq + qi;
    const rtp_bf16 *qr = q_pre + (((size_t)b * g.Hq + h) * g.nq + qi) * kD;
#pragma unroll
    for (int c = 0; c < kD / 32; ++c) {
      const int d0 = 32 * c + 8 * grp;
      const uint4 w = *reinterpret_cast<const uint4 *>(qr + d0);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      float r[8];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        double sn, cs;
        rope_sincos(mq, g.theta, d0 / 2 + pp, sn, cs);
        const double a = (double)bf_lo(ww[pp]), bb = (double)bf_hi(ww[pp]);
        r[2 * pp] = (float)((a * cs - bb * sn) * kQScale);
        r[2 * pp + 1] = (float)((a * sn + bb * cs) * kQScale);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const short hi = bf16_rne(r[e]);
        qh[c][e] = hi;
        ql[c][e] = bf16_rne(r[e] - bf16_f(hi));
      }
    }
  }

  // key blocks: the sink blocks (local heads), then the window or the whole prefix
  const long long lo_pos = dense ? 0 : (m0 - g.window + 1 > 0 ? m0 - g.window + 1 : 0);
  const long long sink_end = dense ? 0 : (g.n_sink < lo_pos ? g.n_sink : lo_pos);   // sink positions [0, sink_end)
  const long long sb_end = (sink_end + kFk - 1) / kFk;                                 // sink blocks [0, sb_end)
  const long long mb_lo = lo_pos / kFk > sb_end ? lo_pos / kFk : sb_end;
  const long long mb_hi = m_hi / kFk;
  const long long nblk = sb_end + (mb_hi >= mb_lo ? mb_hi - mb_lo + 1 : 0);
  const long long qp = m0 + qn;                                // this lane's query position

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[kD / 16];
#pragma unroll
  for (int t = 0; t < kD / 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // staging: the next block is loaded into registers while this block is
  // computed, then written to LDS once every wave is done with this block
  // (one K/V buffer and two barriers per block: 34 KB of LDS, so three
  // workgroups share a CU, one more than with two buffers).
  // Keys: thread t takes key row t / 4, channels 32 (t % 4) .. + 31.  Values:
  // thread t takes the four keys 4 vq .. + 3 (vq = t % 16) of channels
  // 8 vo .. + 7 (vo = 4 wave + lane / 16) and writes each channel's four keys
  // as one 8-byte word of the transposed block; with the 144-byte row pitch
  // the 32 lanes of a half-wave land on 64 distinct banks.
  const int sr = tid >> 2, spart = tid & 3;
  const int vq = tid & 15, vo = 4 * wv + (lane >> 4);
  uint4 k0v, k1v, k2v, k3v, v0v, v1v, v2v, v3v;               // the next block's slice, in flight
#define RTP_FLASH_LOAD(KB)                                                                       \
  {                                                                                              \
    long long kp = (KB) * kFk + sr;                                                              \
    kp = kp < g.N ? kp : g.N - 1;                                                                \
    const uint4 *ks = reinterpret_cast<const uint4 *>(kc + (cbase + kp) * kD + 32 * spart);     \
    k0v = ks[0]; k1v = ks[1]; k2v = ks[2]; k3v = ks[3];                                          \
    long long vp = (KB) * kFk + 4 * vq;                                                          \
    const long long vl = g.N - 1;                                                                \
    const rtp_bf16 *vs = vc + cbase * kD + 8 * vo;                                               \
    v0v = *reinterpret_cast<const uint4 *>(vs + (vp < vl ? vp : vl) * kD);                       \
    v1v = *reinterpret_cast<const uint4 *>(vs + (vp + 1 < vl ? vp + 1 : vl) * kD);               \
    v2v = *reinterpret_cast<const uint4 *>(vs + (vp + 2 < vl ? vp + 2 : vl) * kD);               \
    v3v = *reinterpret_cast<const uint4 *>(vs + (vp + 3 < vl ? vp + 3 : vl) * kD);               \
  }
  // channel 8 vo + c of the four keys: element c of each row's 16 bytes
  auto store_v = [&](int buf) {
    const uint32_t r0[4] = {v0v.x, v0v.y, v0v.z, v0v.w}, r1[4] = {v1v.x, v1v.y, v1v.z, v1v.w};
    const uint32_t r2[4] = {v2v.x, v2v.y, v2v.z, v2v.w}, r3[4] = {v3v.x, v3v.y, v3v.z, v3v.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint2 ev = {(r0[w] & 0xffffu) | (r1[w] << 16), (r2[w] & 0xffffu) | (r3[w] << 16)};
      const uint2 od = {(r0[w] >> 16) | (r1[w] & 0xffff0000u), (r2[w] >> 16) | (r3[w] & 0xffff0000u)};
      *reinterpret_cast<uint2 *>(&sm.vt[buf][8 * vo + 2 * w][4 * vq]) = ev;
      *reinterpret_cast<uint2 *>(&sm.vt[buf][8 * vo + 2 * w + 1][4 * vq]) = od;
    }
  };
#define RTP_FLASH_STORE(BUF)                                                                     \
  {                                                                                              \
    uint4 *kd = reinterpret_cast<uint4 *>(&sm.k[BUF][sr][32 * spart]);                          \
    kd[0] = k0v; kd[1] = k1v; kd[2] = k2v; kd[3] = k3v;                                          \
    store_v(BUF);                                                                                \
  }
  auto block_of = [&](long long x) { return x < sb_end ? x : mb_lo + (x - sb_end); };
  if (nblk > 0) {
    RTP_FLASH_LOAD(block_of(0));
    RTP_FLASH_STORE(0);
  }
  __syncthreads();

  for (long long x = 0; x < nblk; ++x) {
    const long long kb = block_of(x);
    const int buf = (int)(x % kBufs);
    RTP_FLASH_LOAD(block_of(x + 1 < nblk ? x + 1 : x));       // clamped: the last block reloads itself
    if (has_head) {                                            // wave-uniform
    // S^T for the block's four 16-key subtiles
    f32x4_t s[kFk / 16];
#pragma unroll
    for (int st = 0; st < kFk / 16; ++st) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kD / 32; ++c) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(&sm.k[buf][16 * st + qn][32 * c + 8 * grp]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[c], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[c], acc, 0, 0, 0);
      }
      s[st] = acc;
    }
    // masks (this lane holds query qn and keys 64 kb + 16 st + 4 grp + e), only
    // on blocks that straddle the causal edge, the window's start or the sinks
    const int k0 = (int)(kb * kFk), k1 = k0 + kFk - 1;
    const bool inside = k1 <= (int)m0 &&
                        (dense || k1 < g.n_sink || (long long)k0 > m_hi - g.window);      // block-uniform
    float mb = -INFINITY;
#pragma unroll
    for (int st = 0; st < kFk / 16; ++st) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!inside) {
          const int kp = k0 + 16 * st + 4 * grp + e, q32 = (int)qp;
          const bool ok = kp <= q32 && (dense || kp < g.n_sink || kp > q32 - g.window);
          s[st][e] = ok ? s[st][e] : -INFINITY;
        }
        mb = fmaxf(mb, s[st][e]);
      }
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    // The reference maximum m_run moves only when a score of some query of
    // the wave exceeds it by more than kLazy (wave-uniform branch).  Any
    // reference gives the same o / l: the weights carry a common factor that
    // cancels, and a weight stays below 2^kLazy, so nothing overflows.
    if (__any(mb > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mb);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      // O rows are queries 4 grp + e: their factors come from the lanes holding those queries
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __shfl(alpha, 4 * grp + e);
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) o[t][e] *= ae;
      }
    }
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;       // masked scores: exp2(-inf) = 0
    float ps = 0.f;
    bf16x4_t pb[kFk / 16], pl[kFk / 16];                      // P = hi + lo, both bf16
#pragma unroll
    for (int st = 0; st < kFk / 16; ++st) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(s[st][e] - m_ref);
        ps += pe;
        const short hi = bf16_rne(pe);
        pb[st][e] = hi;
        pl[st][e] = bf16_rne(pe - bf16_f(hi));
      }
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run += ps;
    // O += P V in K = 32 steps over subtile pairs (2 j, 2 j + 1): slot 8 grp + e
    // of a step is key 16 (2 j) + 4 grp + e and slot 8 grp + 4 + e is key
    // 16 (2 j + 1) + 4 grp + e, the same order for P and for V
    bf16x8_t ph[kFk / 32], plo[kFk / 32];
#pragma unroll
    for (int j = 0; j < kFk / 32; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ph[j][e] = pb[2 * j][e];
        ph[j][4 + e] = pb[2 * j + 1][e];
        plo[j][e] = pl[2 * j][e];
        plo[j][4 + e] = pl[2 * j + 1][e];
      }
    }
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) {
#pragma unroll
      for (int j = 0; j < kFk / 32; ++j) {
        const bf16x4_t v0 = *reinterpret_cast<const bf16x4_t *>(&sm.vt[buf][16 * t + qn][32 * j + 4 * grp]);
        const bf16x4_t v1 = *reinterpret_cast<const bf16x4_t *>(&sm.vt[buf][16 * t + qn][32 * j + 16 + 4 * grp]);
        const bf16x8_t bv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[j], bv, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[j], bv, o[t], 0, 0, 0);
      }
    }
    }                                                          // has_head
    if (kBufs == 1) __syncthreads();                           // every wave is done with the block
    if (x + 1 < nblk) RTP_FLASH_STORE((int)((x + 1) % kBufs));
    __syncthreads();
  }
#undef RTP_FLASH_LOAD
#undef RTP_FLASH_STORE
  if (!has_head) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int qe = 4 * grp + e;
    const float le = __shfl(l_run, qe);
    if (qe < nqt) {
      float *dst = out + (((size_t)b * g.Hq + h) * g.nq + i0 + qe) * kD + qn;
#pragma unroll
      for (int t = 0; t < kD / 16; ++t) dst[16 * t] = o[t][e] / le;
    }
  }
}

}  // namespace

// Head quads: up to four q heads of one KV group and one mode per workgroup;
// dense quads in fq[1], window + sinks quads in fq[0].
int make_flash_quads(const Geo &g, bool all_dense, FlashQuads fq[2]) {
  memset(fq, 0, 2 * sizeof(FlashQuads));
  for (int kv = 0; kv < g.Hkv; ++kv) {
    for (int mode = 1; mode >= 0; --mode) {
      FlashQuads &f = fq[mode];
      int cnt = 0;
      for (int h = kv * g.G; h < (kv + 1) * g.G; ++h) {
        const bool local = (g.lmask[h >> 5] >> (h & 31)) & 1u;
        const int hm = (all_dense || !local) ? 1 : 0;
        if (hm != mode) continue;
        if (cnt % 4 == 0) {
          if (f.n >= kMaxQuads) return RTP_ERR_UNSUPPORTED;
          f.dense[f.n] = (uint8_t)mode;
          ++f.n;
        }
        RTP_HOST_CHECK(f.n >= 1 && f.n <= kMaxQuads && h < g.Hq && h <= 255);
        f.head[4 * (f.n - 1) + cnt % 4] = (uint8_t)h;
        f.nh[f.n - 1] = (uint8_t)(cnt % 4 + 1);
        ++cnt;
      }
    }
  }
  RTP_HOST_CHECK(fq[0].n + fq[1].n <= kMaxQuads * 2);
  return RTP_OK;
}

static_assert(sizeof(Geo) + sizeof(FlashQuads) + 5 * sizeof(void *) + sizeof(int) <= 4096,
              "kernel arguments beyond the 4 KiB argument segment");

// The dense quads and the window quads go in two launches: in one launch, the
// long dense workgroups and the short window workgroups were measured to run
// three times slower than the two launches back to back.
int launch_flash_prefill(const Geo &g, const FlashQuads fq[2], const rtp_bf16 *q_pre, const rtp_bf16 *k,
                         const rtp_bf16 *v, float *out, hipStream_t s) {
  const int ntiles = (g.nq + kFq - 1) / kFq;
  for (int mode = 1; mode >= 0; --mode) {
    if (fq[mode].n == 0) continue;
    const long long grid = (long long)(ntiles + 7) / 8 * 8 * fq[mode].n * g.B;
    hipLaunchKernelGGL(flash_prefill_kernel, dim3((unsigned)grid), dim3(kWG), 0, s, g, fq[mode], q_pre, k, v, out,
                       ntiles);
    if (hipGetLastError() != hipSuccess) return RTP_ERR_HIP;
  }
  return RTP_OK;
}

}  // namespace rtp
