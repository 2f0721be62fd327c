// C entry points of librtp.so: argument validation, workspace layout, launch.
// The operations and their sources are documented in include/rtp.h.
#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "rtp_internal.h"

namespace rtp {
namespace {

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  Geo g;
  size_t ws_bytes;
  size_t header_bytes;      // the persistent state at the workspace's start (left zero by every call)
};

int count_retrieval(const rtp_layer *L) {
  int hr = 0;
  for (int h = 0; h < L->Hq; ++h) hr += L->head_mode[h] ? 1 : 0;
  return hr;
}

int validate_layer(const rtp_layer *L) {
  if (!L || !L->head_mode) return RTP_ERR_ARG;
  if (L->D != kD || L->R != kR) return RTP_ERR_SHAPE;
  if (L->B < 1 || L->Hq < 1 || L->Hkv < 1 || L->Hq > kMaxHq || L->Hq % L->Hkv != 0) return RTP_ERR_SHAPE;
  if (L->nq < 1 || L->N < L->nq || L->N > L->Ncap || L->N >= (1ll << 31)) return RTP_ERR_SHAPE;
  if ((int64_t)L->B * L->Hq * L->nq >= (1ll << 31)) return RTP_ERR_SHAPE;     // (b, head, query) units in an int
  if (!(L->p > 0.0) || L->window < 1 || L->n_sink < 0 || !(L->rope_theta > 0.0)) return RTP_ERR_ARG;
  for (int h = 0; h < L->Hq; ++h)
    if (L->head_mode[h] != 0 && L->head_mode[h] != 1) return RTP_ERR_ARG;
  const int G = L->Hq / L->Hkv;
  if (L->idx_group < 0 || (L->idx_group > 1 && L->idx_group != G)) return RTP_ERR_ARG;
  if (L->top_k < 0) return RTP_ERR_ARG;
  if (L->local_ring != 0 && L->local_ring != 1) return RTP_ERR_ARG;
  if (L->local_ring && (int64_t)L->n_sink + L->window >= (1ll << 31)) return RTP_ERR_ARG;   // ring rows < 2^31
  if (L->scan_tile != 0 && L->scan_tile != 1024 && L->scan_tile != 2048 && L->scan_tile != 4096 &&
      L->scan_tile != 8192)
    return RTP_ERR_ARG;
  if (L->swa_chunk < 0 || L->swa_chunk % 64 != 0 || L->pf_qch < 0 || L->pf_qch % 16 != 0) return RTP_ERR_ARG;
  if (L->idx_group > 1)        // shared indexer keys: retrieval heads come in whole KV groups
    for (int kv = 0; kv < L->Hkv; ++kv)
      for (int h = kv * G + 1; h < (kv + 1) * G; ++h)
        if (L->head_mode[h] != L->head_mode[kv * G]) return RTP_ERR_ARG;
  return RTP_OK;
}

// Workgroups the GPU holds at once for the decode kernels: 256 CUs x 4
// (each kernel is built for 128 VGPRs and at most 40 KB of LDS).
constexpr long long kSlots = 1024;

int pick_tile(long long N, int forced) {
  if (forced) return forced;
  // The largest tile that still gives four tiles per query, up to 8192
  // positions: fewer, longer tiles mean fewer tile summaries and prefix
  // entries for the selection launch (measured at 1M: phase A 102.8 us at
  // 8192 against 106.4 at 4096 and 134.3 at 2048; at 128K 8192 is best too).
  int T = 1024;
  while (T < 8192 && 4 * T <= N) T *= 2;
  return T;
}

// Geometry of a call (tiling, split counts; no memory).
// dense: the comparator's plan -- every head attends like a local head over a
// window covering the whole cache with no sinks, in chunks of about 2048
// workgroups in total.
int make_geo(const rtp_layer *L, bool dense, Geo &g) {
  const int st = validate_layer(L);
  if (st != RTP_OK) return st;
  int8_t all_local[kMaxHq];
  rtp_layer LD;
  if (dense) {
    memset(all_local, 0, sizeof(all_local));
    LD = *L;
    LD.head_mode = all_local;
    LD.window = (int32_t)(L->N < 0x7fffffff ? L->N : 0x7fffffff);
    LD.n_sink = 0;
    LD.idx_group = 1;
    LD.local_ring = 0;
    L = &LD;
  }
  memset(&g, 0, sizeof(g));
  g.cstride = 1;
  g.B = L->B;
  g.Hq = L->Hq;
  g.Hkv = L->Hkv;
  g.G = L->Hq / L->Hkv;
  g.nq = L->nq;
  g.N = L->N;
  g.Ncap = L->Ncap;
  g.p = L->p;
  g.topk = L->top_k;
  g.window = L->window;
  g.n_sink = L->n_sink;
  g.theta = L->rope_theta;
  int hr = 0, max_local = 0;
  for (int h = 0; h < L->Hq; ++h) {
    if (L->head_mode[h]) g.rhead[hr++] = (uint8_t)h;
    else g.lmask[h >> 5] |= 1u << (h & 31);
  }
  g.Hr = hr;
  g.ig = L->idx_group > 1 ? L->idx_group : 1;
  g.Hi = hr / g.ig;
  for (int kv = 0; kv < L->Hkv; ++kv) {
    int nl = 0;
    for (int h = kv * g.G; h < (kv + 1) * g.G; ++h) nl += L->head_mode[h] ? 0 : 1;
    if (nl) g.lgroup[g.nlg++] = (uint8_t)kv;
    if (nl > max_local) max_local = nl;
    if (L->local_ring && nl == g.G) g.gring[kv >> 5] |= 1u << (kv & 31);
  }
  {
    int nring = 0;
    for (int w = 0; w < kMaxHq / 32; ++w) nring += __builtin_popcount(g.gring[w]);
    g.any_ring = nring > 0;
    g.rows_b = (long long)(g.Hkv - nring) * g.Ncap + (long long)nring * ((long long)g.n_sink + g.window);
  }
  g.units = g.B * g.Hr * g.nq;
  g.T = pick_tile(g.N, L->scan_tile);
  g.nt = (int)((g.N + g.T - 1) / g.T);
  {
    // about 512 selection workgroups, each over at most 16K positions (their
    // codes are staged in LDS)
    long long per = (long long)g.units * g.N / 512;
    int tpw = 1;
    while (tpw * 2 <= 16384 / g.T && (long long)tpw * 2 * g.T <= per) tpw *= 2;
    g.fin_tpw = tpw;
    g.fin_nwg = (g.nt + tpw - 1) / tpw;
  }
  g.swa_units = g.B * g.nlg * g.nq;
  g.swa_hb = (max_local + kSwaHeads - 1) / kSwaHeads;
  {
    const long long lo = g.N - 1 - g.window + 1 > 0 ? g.N - g.window : 0;
    const long long ns = g.n_sink < lo ? g.n_sink : lo;
    const long long Lrows = ns + (g.N - lo);
    long long chunk = (Lrows + 15) / 16;
    // when the scan tiles leave room in one round of workgroups, smaller
    // window chunks fill it (more rows in flight at once; measured at 128K)
    const long long n_scan = (long long)g.units * g.nt, per_chunk = (long long)g.B * g.nlg * g.nq * g.swa_hb;
    if (!dense && per_chunk > 0 && n_scan < kSlots) {
      const long long nch = (kSlots - n_scan) / per_chunk;
      if (nch > 16) chunk = (Lrows + nch - 1) / nch;
    }
    chunk = (chunk + 31) / 32 * 32;
    if (chunk < 64) chunk = 64;
    if (dense) {
      const long long per = (long long)g.swa_units * g.swa_hb * Lrows / 2048;
      chunk = per < 1024 ? 1024 : (per + 63) / 64 * 64;
      if (chunk > (1ll << 30)) chunk = 1ll << 30;     // huge layers: the row count stays an int
    }
    if (L->swa_chunk) chunk = L->swa_chunk;
    g.swa_chunk = (int)chunk;
    g.swa_nch = (int)((Lrows + chunk - 1) / chunk);
    RTP_HOST_CHECK(g.swa_chunk >= 64 && g.swa_chunk % 32 == 0);
    RTP_HOST_CHECK((long long)g.swa_nch * g.swa_chunk >= Lrows && (long long)(g.swa_nch - 1) * g.swa_chunk < Lrows);
  }
#ifdef RTP_HOST_CHECKS
  {
    int nloc = 0;
    for (int w = 0; w < kMaxHq / 32; ++w) nloc += __builtin_popcount(g.lmask[w]);
    RTP_HOST_CHECK(g.Hr + nloc == g.Hq);
  }
  for (int r = 0; r < g.Hr; ++r) RTP_HOST_CHECK(g.rhead[r] < g.Hq && L->head_mode[g.rhead[r]] == 1);
  for (int j = 0; j < g.nlg; ++j) RTP_HOST_CHECK(g.lgroup[j] < g.Hkv);
#endif
  RTP_HOST_CHECK(g.Hi * g.ig == g.Hr && g.nlg <= g.Hkv && g.swa_hb * kSwaHeads >= max_local);
  RTP_HOST_CHECK(g.T >= 1024 && g.T <= 8192 && (g.T & (g.T - 1)) == 0);
  RTP_HOST_CHECK((long long)g.nt * g.T >= g.N && (long long)(g.nt - 1) * g.T < g.N);
  RTP_HOST_CHECK(g.fin_tpw >= 1 && (g.fin_tpw & (g.fin_tpw - 1)) == 0 && (long long)g.fin_tpw * g.T <= 16384);
  RTP_HOST_CHECK((long long)g.fin_nwg * g.fin_tpw >= g.nt && (long long)(g.fin_nwg - 1) * g.fin_tpw < g.nt);
  // every launch's workgroup count fits the grid's 32-bit x dimension
  const long long n_scan = (long long)g.units * g.nt, n_fin = (long long)g.units * g.fin_nwg;
  const long long n_swa = (long long)g.swa_units * g.swa_hb * g.swa_nch;
  if (n_scan + n_swa >= (1ll << 31) || n_fin + (long long)g.swa_units * g.swa_hb >= (1ll << 31))
    return RTP_ERR_UNSUPPORTED;
  return RTP_OK;
}

// Geometry and workspace layout of a call; ws may be null (sizing only).
// The workspace starts with the state every call leaves zeroed for the next
// one (merge ring, cell ranges, arrival counters).  Its layout depends only on
// B, Hq, Hkv, nq and head_mode -- not on N, so a growing decode cache keeps
// using one workspace -- and is shared by the step's plan and the dense
// comparator's plan, whose transient regions follow it.
int make_plan(const rtp_layer *L, void *ws, Plan *out, bool dense = false) {
  Geo reg, den;
  int st = make_geo(L, false, reg);
  if (st != RTP_OK) return st;
  st = make_geo(L, true, den);
  if (st != RTP_OK) return st;
  Geo g = dense ? den : reg;
  size_t off = 0;
  const size_t units = (size_t)g.units, nt = (size_t)g.nt;
  const size_t reg_units = (size_t)reg.units;
  const size_t swa_ctrs = std::max((size_t)reg.swa_units * reg.swa_hb, (size_t)den.swa_units * den.swa_hb);
  const size_t o_ring = off;
  off = align_up(off + reg_units * kRing * 8);
  // control words one 256-byte line apart for decode (few queries, many
  // workgroups per query); packed for chunked prefill (many queries)
  const size_t cs = g.nq == 1 ? 64 : 1;
  g.cstride = (int)cs;
  const size_t o_cmax = off;
  off = align_up(off + reg_units * cs * 4);
  const size_t o_cmin = off;
  off = align_up(off + reg_units * cs * 4);
  const size_t o_ctr_fin = off;
  off = align_up(off + reg_units * cs * 4);
  const size_t o_ctr_swa = off;
  off = align_up(off + swa_ctrs * cs * 4);
  // transient regions of this call
  const size_t o_qprep = off;
  out->header_bytes = off;
  off = align_up(off + units * sizeof(QPrep));
  const size_t o_tsum = off;
  off = align_up(off + units * nt * sizeof(TileSum));
  const size_t o_part = off;
  off = align_up(off + units * (nt > (size_t)kSpChunks ? nt : (size_t)kSpChunks) * sizeof(Partial));  // >= fin_nwg
  const size_t o_swa = off;
  off = align_up(off + (size_t)g.swa_units * g.swa_hb * g.swa_nch * kSwaHeads * sizeof(Partial));

  // the codes of the decode path and, for nq > 1, the chunked prefill's
  // selected positions (never used by the same call) share one region
  g.pf_qch = 0;
  size_t pf_idx_bytes = 0, pf_cnt_bytes = 0;
  if (g.nq > 1 && g.units > 0) {
    const long long per_q = (long long)g.B * g.Hr * g.N * 4;      // bytes of positions per query index
    long long qch = (8ll << 30) / per_q;                            // up to 8 GiB of positions per chunk
    qch = qch / 16 * 16;
    if (L->pf_qch) qch = L->pf_qch;
    if (qch < 16) qch = 16;
    if (qch > g.nq) qch = g.nq;
    g.pf_qch = (int)qch;
    pf_idx_bytes = align_up((size_t)qch * per_q);
    pf_cnt_bytes = align_up((size_t)g.B * g.Hr * qch * 4);
  }
  const size_t o_codes = off;
  {
    const size_t codes_bytes = units * nt * (size_t)g.T;
    const size_t pf_bytes = pf_idx_bytes + pf_cnt_bytes;
    off = align_up(off + (codes_bytes > pf_bytes ? codes_bytes : pf_bytes));
  }
  // regions in order, each inside the workspace and 256-byte aligned
  RTP_HOST_CHECK(o_ring == 0 && o_cmax >= o_ring + reg_units * kRing * 8 && o_cmin >= o_cmax + reg_units * cs * 4);
  RTP_HOST_CHECK(o_ctr_fin >= o_cmin + reg_units * cs * 4 && o_ctr_swa >= o_ctr_fin + reg_units * cs * 4);
  RTP_HOST_CHECK(o_qprep >= o_ctr_swa + swa_ctrs * cs * 4 && o_tsum >= o_qprep + units * sizeof(QPrep));
  RTP_HOST_CHECK(o_part >= o_tsum + units * nt * sizeof(TileSum));
  RTP_HOST_CHECK(o_swa >= o_part + units * (size_t)std::max(g.fin_nwg, kSpChunks) * sizeof(Partial));
  RTP_HOST_CHECK(o_codes >= o_swa + (size_t)g.swa_units * g.swa_hb * g.swa_nch * kSwaHeads * sizeof(Partial));
  RTP_HOST_CHECK(off >= o_codes + units * nt * (size_t)g.T && off >= o_codes + pf_idx_bytes + pf_cnt_bytes);
  RTP_HOST_CHECK(g.nq == 1 || g.units == 0 ||
                 (g.pf_qch >= 1 && g.pf_qch <= g.nq &&
                  pf_idx_bytes >= (size_t)g.pf_qch * g.B * g.Hr * (size_t)g.N * 4 &&
                  pf_cnt_bytes >= (size_t)g.B * g.Hr * g.pf_qch * 4));
#ifdef RTP_HOST_CHECKS
  for (size_t o : {o_ring, o_cmax, o_cmin, o_ctr_fin, o_ctr_swa, o_qprep, o_tsum, o_part, o_swa, o_codes, off})
    RTP_HOST_CHECK(o % 256 == 0);
#endif
  // the persistent header does not depend on N: the dense plan's counters fit it too
  RTP_HOST_CHECK((size_t)den.swa_units * den.swa_hb <= swa_ctrs && den.units == 0);
  if (ws) {
    char *base = static_cast<char *>(ws);
    g.ring = reinterpret_cast<uint64_t *>(base + o_ring);
    g.cmax = reinterpret_cast<uint32_t *>(base + o_cmax);
    g.cmin = reinterpret_cast<uint32_t *>(base + o_cmin);
    g.ctr_fin = reinterpret_cast<uint32_t *>(base + o_ctr_fin);
    g.ctr_swa = reinterpret_cast<uint32_t *>(base + o_ctr_swa);
    g.tsum = reinterpret_cast<TileSum *>(base + o_tsum);
    g.qprep = reinterpret_cast<QPrep *>(base + o_qprep);
    g.part = reinterpret_cast<Partial *>(base + o_part);
    g.swa_part = reinterpret_cast<Partial *>(base + o_swa);
    g.codes = reinterpret_cast<uint8_t *>(base + o_codes);
    g.pf_idx = reinterpret_cast<int32_t *>(base + o_codes);
    g.pf_cnt = reinterpret_cast<int32_t *>(base + o_codes + pf_idx_bytes);
  }
  out->g = g;
  out->ws_bytes = off;
  return RTP_OK;
}

bool has_ring(const Geo &g) { return g.any_ring != 0; }

// The kernels access every device array with 16-byte vector loads and
// stores; null pointers count as aligned (their calls check them apart).
bool aligned16(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  return true;
}

int plan_with_ws(const rtp_layer *L, void *ws, size_t ws_bytes, Plan *p, bool dense = false) {
  const int st = make_plan(L, ws, p, dense);
  if (st != RTP_OK) return st;
  if (!ws) return RTP_ERR_ARG;
  if (ws_bytes < p->ws_bytes) return RTP_ERR_WS_TOO_SMALL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return RTP_ERR_ARG;
  return RTP_OK;
}

// Cluster-index scratch after the regular workspace; ws may be null (sizing).
int cluster_plan(const rtp_layer *L, int K, void *ws, Geo *g_out, ClGeo *cg, size_t *bytes) {
  Plan p, pd;
  int st = make_plan(L, ws, &p);
  if (st != RTP_OK) return st;
  st = make_plan(L, nullptr, &pd, true);
  if (st != RTP_OK) return st;
  if (K < 1 || K > kMaxClusters || K > L->N) return RTP_ERR_ARG;
  const Geo &g = p.g;
  const size_t nu = (size_t)g.B * g.Hi, units = (size_t)g.units;
  const int ntiles = (int)((g.N + cluster_tile() - 1) / cluster_tile());
  size_t off = align_up(p.ws_bytes > pd.ws_bytes ? p.ws_bytes : pd.ws_bytes);
  const size_t o_sum = off;
  off = align_up(off + nu * K * kR * sizeof(double));
  const size_t o_cnt = off;
  off = align_up(off + nu * K * 4);
  const size_t o_assign = off;
  off = align_up(off + nu * (size_t)g.N * 4);
  const size_t o_hist = off;
  off = align_up(off + nu * (size_t)ntiles * K * 4);
  const size_t o_start = off;
  off = align_up(off + units * K * 4);
  const size_t o_total = off;
  off = align_up(off + units * 4);
  const size_t o_list = off;
  off = align_up(off + units * (size_t)g.N * 4);
  memset(cg, 0, sizeof(*cg));
  cg->K = K;
  cg->ntiles = ntiles;
  if (ws) {
    char *base = static_cast<char *>(ws);
    cg->sum = reinterpret_cast<double *>(base + o_sum);
    cg->cnt = reinterpret_cast<uint32_t *>(base + o_cnt);
    cg->assign = reinterpret_cast<int32_t *>(base + o_assign);
    cg->hist = reinterpret_cast<uint32_t *>(base + o_hist);
    cg->start = reinterpret_cast<int32_t *>(base + o_start);
    cg->total = reinterpret_cast<int32_t *>(base + o_total);
    cg->list = reinterpret_cast<int32_t *>(base + o_list);
  }
  *g_out = g;
  *bytes = off;
  return RTP_OK;
}

// The launch wrappers report failures through hipGetLastError(); clear an
// error left by earlier, unrelated runtime calls so it is not taken for ours.
hipStream_t as_stream(void *s) {
  (void)hipGetLastError();
  return reinterpret_cast<hipStream_t>(s);
}

}  // namespace
}  // namespace rtp

// ---------------------------------------------------------------- the allocation-free step
// rtp_decode_step_static's scratch: one array per GPU.  Host code never uses the array's name as an address; the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[RTP_STATIC_SCRATCH_BYTES];

namespace rtp {
namespace {
struct StaticScratch {
  void *ptr = nullptr;           // device address of `scratch` on this device
  size_t key_hash = 0;           // layout of the persistent header the last call left zero
  size_t header_bytes = 0;
  bool used = false;
};
constexpr int kMaxDevices = 64;
StaticScratch g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Layout key of the persistent header: it depends on B, Hq, Hkv, nq and head_mode.
size_t header_key(const rtp_layer *L) {
  size_t h = 1469598103934665603ull;
  auto mix = [&](long long v) { h = (h ^ (size_t)v) * 1099511628211ull; };
  mix(L->B);
  mix(L->Hq);
  mix(L->Hkv);
  mix(L->nq);
  for (int i = 0; i < L->Hq; ++i) mix(L->head_mode[i]);
  return h;
}
}  // namespace
}  // namespace rtp

using namespace rtp;

extern "C" {

const char *rtp_status_str(int status) {
  switch (status) {
    case RTP_OK: return "ok";
    case RTP_ERR_ARG: return "invalid argument";
    case RTP_ERR_SHAPE: return "unsupported or inconsistent shape";
    case RTP_ERR_WS_TOO_SMALL: return "workspace too small";
    case RTP_ERR_UNSUPPORTED: return "not supported by this library";
    case RTP_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t rtp_num_retrieval(const rtp_layer *layer) {
  const int st = validate_layer(layer);
  return st != RTP_OK ? st : count_retrieval(layer);
}

int64_t rtp_kv_rows(const rtp_layer *layer) {
  Geo g;
  const int st = make_geo(layer, false, g);
  return st != RTP_OK ? st : g.rows_b;
}

size_t rtp_workspace_bytes(const rtp_layer *layer) {
  Plan p, pd;
  if (make_plan(layer, nullptr, &p) != RTP_OK || make_plan(layer, nullptr, &pd, true) != RTP_OK) return 0;
  return p.ws_bytes > pd.ws_bytes ? p.ws_bytes : pd.ws_bytes;
}

int rtp_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws) return RTP_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return RTP_ERR_ARG;
  return launch_fill_zero(ws, ws_bytes, as_stream(stream));
}

int rtp_rope_keys(const rtp_layer *layer, const rtp_bf16 *k_pre, rtp_bf16 *k_out, int64_t n0, int64_t n1,
                  void *stream) {
  Plan p;
  int st = make_plan(layer, nullptr, &p);
  if (st != RTP_OK) return st;
  if (!k_pre || !k_out || n0 < 0 || n1 < n0 || n1 > layer->Ncap) return RTP_ERR_ARG;
  if (!aligned16({k_pre, k_out})) return RTP_ERR_ARG;
  return launch_rope_keys(p.g, k_pre, k_out, n0, n1, as_stream(stream));
}

int rtp_index_keys(const rtp_layer *layer, const rtp_bf16 *k_pre, const rtp_bf16 *w_k, rtp_bf16 *k_idx, int64_t n0,
                   int64_t n1, void *stream) {
  Plan p;
  int st = make_plan(layer, nullptr, &p);
  if (st != RTP_OK) return st;
  if (!k_pre || !w_k || !k_idx || n0 < 0 || n1 < n0 || n1 > layer->Ncap) return RTP_ERR_ARG;
  if (!aligned16({k_pre, w_k, k_idx})) return RTP_ERR_ARG;
  return launch_index_keys(p.g, k_pre, w_k, k_idx, n0, n1, as_stream(stream));
}

int rtp_index_score(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                    float *logits, void *stream) {
  Plan p;
  int st = make_plan(layer, nullptr, &p);
  if (st != RTP_OK) return st;
  if (p.g.units && (!q_pre || !w_q || !k_idx || !logits)) return RTP_ERR_ARG;
  if (!aligned16({q_pre, w_q, k_idx, logits})) return RTP_ERR_ARG;
  return launch_index_score(p.g, q_pre, w_q, k_idx, logits, as_stream(stream));
}

int rtp_topp_select(const rtp_layer *layer, const float *logits, int32_t *idx, int32_t *count, int64_t cap, void *ws,
                    size_t ws_bytes, void *stream) {
  Plan p;
  int st = plan_with_ws(layer, ws, ws_bytes, &p);
  if (st != RTP_OK) return st;
  if (p.g.units && (!logits || !count || cap < 0 || (cap > 0 && !idx))) return RTP_ERR_ARG;
  if (!aligned16({logits, idx, count})) return RTP_ERR_ARG;
  hipStream_t s = as_stream(stream);
  st = launch_phase_a(p.g, nullptr, nullptr, nullptr, logits, nullptr, nullptr, nullptr, true, false, s);
  if (st != RTP_OK) return st;
  return launch_finish(p.g, nullptr, logits, nullptr, nullptr, nullptr, cap > 0 ? idx : nullptr,
                       count, cap, s);
}

int rtp_sparse_attn(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *k, const rtp_bf16 *v,
                    const int32_t *idx, const int32_t *count, int64_t cap, float *out, void *ws, size_t ws_bytes,
                    void *stream) {
  Plan p;
  int st = plan_with_ws(layer, ws, ws_bytes, &p);
  if (st != RTP_OK) return st;
  if (p.g.units && (!q_pre || !k || !v || !count || !out || cap < 0 || (cap > 0 && !idx))) return RTP_ERR_ARG;
  if (!aligned16({q_pre, k, v, idx, count, out})) return RTP_ERR_ARG;
  return launch_sparse_attn(p.g, q_pre, k, v, idx, count, cap, out, as_stream(stream));
}

int rtp_swa_attn(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *k, const rtp_bf16 *v, float *out,
                 void *ws, size_t ws_bytes, void *stream) {
  Plan p;
  int st = plan_with_ws(layer, ws, ws_bytes, &p);
  if (st != RTP_OK) return st;
  if (p.g.swa_units && (!q_pre || !k || !v || !out)) return RTP_ERR_ARG;
  if (!aligned16({q_pre, k, v, out})) return RTP_ERR_ARG;
  if (has_ring(p.g) && p.g.nq > 1) return RTP_ERR_UNSUPPORTED;     // a ring holds the newest window only
  return launch_phase_a(p.g, q_pre, nullptr, nullptr, nullptr, k, v, out, false, true, as_stream(stream));
}

int rtp_dense_attn(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *k, const rtp_bf16 *v, float *out,
                   void *ws, size_t ws_bytes, void *stream) {
  Plan p;
  int st = plan_with_ws(layer, ws, ws_bytes, &p, true);
  if (st != RTP_OK) return st;
  if (!q_pre || !k || !v || !out) return RTP_ERR_ARG;
  if (!aligned16({q_pre, k, v, out})) return RTP_ERR_ARG;
  if (layer->local_ring) {                    // every head needs every position
    Geo reg;
    st = make_geo(layer, false, reg);
    if (st != RTP_OK) return st;
    if (has_ring(reg)) return RTP_ERR_UNSUPPORTED;
  }
  if (layer->nq > 1) {            // many queries: the matrix-core kernel, every head dense
    FlashQuads fq[2];
    st = make_flash_quads(p.g, true, fq);
    if (st != RTP_OK) return st;
    return launch_flash_prefill(p.g, fq, q_pre, k, v, out, as_stream(stream));
  }
  return launch_phase_a(p.g, q_pre, nullptr, nullptr, nullptr, k, v, out, false, true, as_stream(stream));
}

int rtp_prefill_attn(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *k, const rtp_bf16 *v, float *out,
                     int32_t all_dense, void *stream) {
  Plan p;
  int st = make_plan(layer, nullptr, &p);
  if (st != RTP_OK) return st;
  if (!q_pre || !k || !v || !out) return RTP_ERR_ARG;
  if (!aligned16({q_pre, k, v, out})) return RTP_ERR_ARG;
  if (has_ring(p.g)) return RTP_ERR_UNSUPPORTED;     // earlier queries need rows a ring no longer holds
  FlashQuads fq[2];
  st = make_flash_quads(p.g, all_dense != 0, fq);
  if (st != RTP_OK) return st;
  return launch_flash_prefill(p.g, fq, q_pre, k, v, out, as_stream(stream));
}

int rtp_append_kv(const rtp_layer *layer, const rtp_bf16 *k_new, const rtp_bf16 *v_new, const rtp_bf16 *w_k,
                  rtp_bf16 *k_cache, rtp_bf16 *v_cache, rtp_bf16 *k_idx, int64_t n0, int64_t n_new, void *stream) {
  Plan p;
  int st = make_plan(layer, nullptr, &p);
  if (st != RTP_OK) return st;
  if (n0 < 0 || n_new < 0 || n0 > layer->Ncap - n_new || n0 + n_new >= (1ll << 31)) return RTP_ERR_ARG;
  if (n_new == 0) return RTP_OK;
  if (!k_new || !v_new || !k_cache || !v_cache) return RTP_ERR_ARG;
  if (p.g.Hi && (!w_k || !k_idx)) return RTP_ERR_ARG;
  if (!aligned16({k_new, v_new, w_k, k_cache, v_cache, k_idx})) return RTP_ERR_ARG;
  return launch_append_kv(p.g, k_new, v_new, w_k, k_cache, v_cache, k_idx, n0, n_new, as_stream(stream));
}

size_t rtp_cluster_workspace_bytes(const rtp_layer *layer, int32_t K) {
  Geo g;
  ClGeo cg;
  size_t bytes = 0;
  return cluster_plan(layer, K, nullptr, &g, &cg, &bytes) == RTP_OK ? bytes : 0;
}

int rtp_cluster_build(const rtp_layer *layer, const rtp_bf16 *k_idx, int32_t K, int32_t iters, rtp_bf16 *centroids,
                      int32_t *counts, int32_t *offsets, int32_t *members, void *ws, size_t ws_bytes, void *stream) {
  Geo g;
  ClGeo cg;
  size_t need = 0;
  int st = cluster_plan(layer, K, ws, &g, &cg, &need);
  if (st != RTP_OK) return st;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return RTP_ERR_ARG;
  if (ws_bytes < need) return RTP_ERR_WS_TOO_SMALL;
  if (iters < 0 || g.Hi == 0 || !k_idx || !centroids || !counts || !offsets || !members) return RTP_ERR_ARG;
  if (!aligned16({k_idx, centroids, counts, offsets, members})) return RTP_ERR_ARG;
  return launch_cluster_build(g, cg, k_idx, iters, centroids, counts, offsets, members, as_stream(stream));
}

int rtp_cluster_step(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, int32_t K,
                     const rtp_bf16 *centroids, const int32_t *counts, const int32_t *offsets, const int32_t *members,
                     const rtp_bf16 *k, const rtp_bf16 *v, float *out, int32_t *idx_opt, int32_t *count_opt,
                     int64_t cap, void *ws, size_t ws_bytes, void *stream) {
  Geo g;
  ClGeo cg;
  size_t need = 0;
  int st = cluster_plan(layer, K, ws, &g, &cg, &need);
  if (st != RTP_OK) return st;
  if (layer->nq != 1 || layer->top_k != 0) return RTP_ERR_UNSUPPORTED;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return RTP_ERR_ARG;
  if (ws_bytes < need) return RTP_ERR_WS_TOO_SMALL;
  if (!q_pre || !k || !v || !out) return RTP_ERR_ARG;
  if (g.units && (!w_q || !centroids || !counts || !offsets || !members)) return RTP_ERR_ARG;
  if (idx_opt && cap < 0) return RTP_ERR_ARG;
  if (!aligned16({q_pre, w_q, centroids, counts, offsets, members, k, v, out, idx_opt, count_opt})) return RTP_ERR_ARG;
  hipStream_t s = as_stream(stream);
  st = launch_phase_a(g, q_pre, nullptr, nullptr, nullptr, k, v, out, false, true, s);      // local heads
  if (st != RTP_OK) return st;
  st = launch_cluster_select(g, cg, q_pre, w_q, centroids, counts, offsets, members, idx_opt, count_opt,
                             idx_opt ? cap : 0, s);
  if (st != RTP_OK) return st;
  return launch_sparse_attn(g, q_pre, k, v, cg.list, cg.total, g.N, out, s);
}

int rtp_decode_step(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                    const rtp_bf16 *k, const rtp_bf16 *v, float *out, int32_t *idx_opt, int32_t *count_opt,
                    int64_t cap, void *ws, size_t ws_bytes, void *phase_event, void *stream) {
  Plan p;
  int st = plan_with_ws(layer, ws, ws_bytes, &p);
  if (st != RTP_OK) return st;
  if (!q_pre || !k || !v || !out) return RTP_ERR_ARG;
  if (p.g.units && (!w_q || !k_idx)) return RTP_ERR_ARG;
  if (idx_opt && cap < 0) return RTP_ERR_ARG;
  if (!aligned16({q_pre, w_q, k_idx, k, v, out, idx_opt, count_opt})) return RTP_ERR_ARG;
  hipStream_t s = as_stream(stream);
  if (layer->nq > 1) {
    if (has_ring(p.g)) return RTP_ERR_UNSUPPORTED;   // earlier queries' windows left the ring
    // chunked prefill: matrix-core selection and attention per chunk of queries
    st = launch_pf_qprep(p.g, q_pre, w_q, s);
    if (st != RTP_OK) return st;
    if (phase_event && hipEventRecord(reinterpret_cast<hipEvent_t>(phase_event), s) != hipSuccess) return RTP_ERR_HIP;
    for (int i0 = 0; p.g.units && i0 < p.g.nq; i0 += p.g.pf_qch) {
      const int nqc = p.g.nq - i0 < p.g.pf_qch ? p.g.nq - i0 : p.g.pf_qch;
      st = launch_pf_select(p.g, k_idx, i0, nqc, p.g.pf_idx, p.g.N, p.g.pf_cnt, idx_opt, count_opt,
                            idx_opt ? cap : 0, s);
      if (st != RTP_OK) return st;
      st = launch_pf_attn(p.g, i0, nqc, k, v, p.g.pf_idx, p.g.N, p.g.pf_cnt, out, s);
      if (st != RTP_OK) return st;
    }
    return launch_phase_a(p.g, q_pre, nullptr, nullptr, nullptr, k, v, out, false, true, s);
  }
  // with retrieval heads the selection launch follows; it also merges the
  // local heads' window chunks, which takes that merge off the scan launch
  const bool defer = p.g.units > 0 && p.g.swa_units > 0;
  st = launch_phase_a(p.g, q_pre, w_q, k_idx, nullptr, k, v, out, true, true, s, defer);
  if (st != RTP_OK) return st;
  if (phase_event && hipEventRecord(reinterpret_cast<hipEvent_t>(phase_event), s) != hipSuccess) return RTP_ERR_HIP;
  return launch_finish(p.g, k_idx, nullptr, k, v, out, idx_opt, count_opt, idx_opt ? cap : 0, s, defer);
}

int rtp_decode_step_static(const rtp_layer *layer, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                           const rtp_bf16 *k, const rtp_bf16 *v, float *out, int32_t *idx_opt, int32_t *count_opt,
                           int64_t cap, void *stream) {
  Plan p;
  int st = make_plan(layer, nullptr, &p);
  if (st != RTP_OK) return st;
  const size_t need = rtp_workspace_bytes(layer);
  if (need == 0) return RTP_ERR_ARG;
  if (need > (size_t)RTP_STATIC_SCRATCH_BYTES) return RTP_ERR_WS_TOO_SMALL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RTP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RTP_ERR_UNSUPPORTED;
  void *ws = nullptr;
  bool clear = false;
  size_t clear_bytes = 0;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    StaticScratch &ss = g_scratch[dev];
    if (!ss.ptr) {
      void *ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return RTP_ERR_HIP;
      ss.ptr = ptr;
    }
    // the persistent header must start zero: every call leaves it zero for
    // the next call of the same layout; the first call on a device and a
    // change of layout clear it here
    const size_t key = header_key(layer);
    if (!ss.used || ss.key_hash != key) {
      clear = true;
      clear_bytes = std::max(ss.used ? ss.header_bytes : 0, p.header_bytes);
    }
    ss.used = true;
    ss.key_hash = key;
    ss.header_bytes = p.header_bytes;
    ws = ss.ptr;
  }
  hipStream_t s = as_stream(stream);
  if (clear) {
    st = launch_fill_zero(ws, (clear_bytes + 255) & ~(size_t)255, s);
    if (st != RTP_OK) return st;
  }
  return rtp_decode_step(layer, q_pre, w_q, k_idx, k, v, out, idx_opt, count_opt, cap, ws, need, nullptr, stream);
}

}  // extern "C"
