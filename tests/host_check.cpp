// Host-side checks of librtp's C entry points and planners.
//
// Built by the CPU tests from the library's sources compiled for the host only,
// with AddressSanitizer, UndefinedBehaviorSanitizer and -DRTP_HOST_CHECKS (the
// planners' bounds assertions), then fed the same calls the ctypes tests make.
// No GPU is needed: every call made here fails validation, or only sizes and
// plans, before anything is launched.
//
// stdin, one command per line; stdout, one result line per command:
//   call <name> <field>=<value>... | <arg>...
//       calls entry point <name> with a layer built from the fields
//       (head_mode as comma-separated 0/1) and the arguments: "L" is the
//       layer's address, other tokens are integers (addresses are never
//       dereferenced).  Prints the return value ("s <text>" for a string).
//   quads <Hq> <Hkv> <all_dense> <head_mode as comma-separated 0/1>
//       runs the prefill attention's head-quad planner and prints
//       "<status> <n0> <n1>" then one line per quad: "q <mode> <j> <dense> <nh> <heads...>".
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <iostream>
#include <map>
#include <sstream>
#include <string>
#include <type_traits>
#include <utility>
#include <vector>

#include "rtp_internal.h"

namespace {

template <class T>
T conv(long long v) {
  if constexpr (std::is_pointer_v<T>)
    return reinterpret_cast<T>(static_cast<intptr_t>(v));
  else
    return static_cast<T>(v);
}

template <class R, class... A, size_t... I>
R invoke(R (*f)(A...), const std::vector<long long> &a, std::index_sequence<I...>) {
  return f(conv<A>(a[I])...);
}

template <class R, class... A>
std::string run(R (*f)(A...), const std::vector<long long> &a) {
  if (a.size() != sizeof...(A)) return "argc";
  R r = invoke(f, a, std::index_sequence_for<A...>{});
  if constexpr (std::is_pointer_v<R>)
    return std::string("s ") + (r ? r : "(null)");
  else
    return std::to_string(static_cast<long long>(r));
}

using Runner = std::string (*)(const std::vector<long long> &);

#define RTP_ENTRY(fn) {#fn, [](const std::vector<long long> &a) { return run(fn, a); }}
const std::map<std::string, Runner> kEntries = {
    RTP_ENTRY(rtp_num_retrieval),     RTP_ENTRY(rtp_kv_rows),
    RTP_ENTRY(rtp_workspace_bytes),   RTP_ENTRY(rtp_workspace_init),
    RTP_ENTRY(rtp_status_str),        RTP_ENTRY(rtp_rope_keys),
    RTP_ENTRY(rtp_index_keys),        RTP_ENTRY(rtp_append_kv),
    RTP_ENTRY(rtp_index_score),       RTP_ENTRY(rtp_topp_select),
    RTP_ENTRY(rtp_sparse_attn),       RTP_ENTRY(rtp_swa_attn),
    RTP_ENTRY(rtp_dense_attn),        RTP_ENTRY(rtp_prefill_attn),
    RTP_ENTRY(rtp_decode_step),       RTP_ENTRY(rtp_decode_step_static),
    RTP_ENTRY(rtp_cluster_workspace_bytes), RTP_ENTRY(rtp_cluster_build),
    RTP_ENTRY(rtp_cluster_step),
};
#undef RTP_ENTRY

std::vector<int8_t> parse_modes(const std::string &s) {
  std::vector<int8_t> m;
  std::stringstream ss(s);
  std::string t;
  while (std::getline(ss, t, ',')) m.push_back(static_cast<int8_t>(std::stoi(t)));
  return m;
}

// The caller gives every field; the layer starts zeroed.
void set_field(rtp_layer &L, std::vector<int8_t> &modes, const std::string &k, const std::string &v) {
  if (k == "B") L.B = std::stoi(v);
  else if (k == "Hq") L.Hq = std::stoi(v);
  else if (k == "Hkv") L.Hkv = std::stoi(v);
  else if (k == "D") L.D = std::stoi(v);
  else if (k == "R") L.R = std::stoi(v);
  else if (k == "nq") L.nq = std::stoi(v);
  else if (k == "N") L.N = std::stoll(v);
  else if (k == "Ncap") L.Ncap = std::stoll(v);
  else if (k == "head_mode") modes = parse_modes(v);
  else if (k == "p") L.p = std::strtod(v.c_str(), nullptr);
  else if (k == "window") L.window = std::stoi(v);
  else if (k == "n_sink") L.n_sink = std::stoi(v);
  else if (k == "rope_theta") L.rope_theta = std::strtod(v.c_str(), nullptr);
  else if (k == "idx_group") L.idx_group = std::stoi(v);
  else if (k == "top_k") L.top_k = std::stoll(v);
  else if (k == "local_ring") L.local_ring = std::stoi(v);
  else if (k == "scan_tile") L.scan_tile = std::stoi(v);
  else if (k == "swa_chunk") L.swa_chunk = std::stoi(v);
  else if (k == "pf_qch") L.pf_qch = std::stoi(v);
  else {
    fprintf(stderr, "unknown field %s\n", k.c_str());
    exit(2);
  }
}

std::string do_call(std::istringstream &in) {
  std::string name, tok;
  in >> name;
  rtp_layer L;
  memset(&L, 0, sizeof(L));
  std::vector<int8_t> modes;
  bool args = false;
  std::vector<long long> a;
  std::vector<size_t> layer_args;
  while (in >> tok) {
    if (tok == "|") {
      args = true;
      continue;
    }
    if (!args) {
      const size_t eq = tok.find('=');
      if (eq == std::string::npos) return "bad field";
      set_field(L, modes, tok.substr(0, eq), tok.substr(eq + 1));
    } else if (tok == "L") {
      layer_args.push_back(a.size());          // the layer's address, filled in below
      a.push_back(0);
    } else {
      a.push_back(std::stoll(tok));
    }
  }
  // the head modes live in an exactly sized heap array, so that a planner
  // reading past Hq entries trips AddressSanitizer
  int8_t *hm = modes.empty() ? nullptr : static_cast<int8_t *>(malloc(modes.size()));
  if (hm) memcpy(hm, modes.data(), modes.size());
  L.head_mode = hm;
  rtp_layer *lp = static_cast<rtp_layer *>(malloc(sizeof(rtp_layer)));
  *lp = L;
  for (size_t i : layer_args) a[i] = static_cast<long long>(reinterpret_cast<intptr_t>(lp));
  auto it = kEntries.find(name);
  std::string r = it == kEntries.end() ? "unknown" : it->second(a);
  free(lp);
  free(hm);
  return r;
}

void do_quads(std::istringstream &in) {
  int Hq = 0, Hkv = 0, all_dense = 0;
  std::string ms;
  in >> Hq >> Hkv >> all_dense >> ms;
  const std::vector<int8_t> modes = parse_modes(ms);
  rtp::Geo g;
  memset(&g, 0, sizeof(g));
  g.Hq = Hq;
  g.Hkv = Hkv;
  g.G = Hq / Hkv;
  for (int h = 0; h < Hq; ++h)
    if (!modes[h]) g.lmask[h >> 5] |= 1u << (h & 31);
  rtp::FlashQuads *fq = static_cast<rtp::FlashQuads *>(malloc(2 * sizeof(rtp::FlashQuads)));
  const int st = rtp::make_flash_quads(g, all_dense != 0, fq);
  std::cout << st << " " << fq[0].n << " " << fq[1].n << "\n";
  for (int mode = 0; mode < 2; ++mode)
    for (int j = 0; j < fq[mode].n; ++j) {
      std::cout << "q " << mode << " " << j << " " << int(fq[mode].dense[j]) << " " << int(fq[mode].nh[j]);
      for (int i = 0; i < fq[mode].nh[j]; ++i) std::cout << " " << int(fq[mode].head[4 * j + i]);
      std::cout << "\n";
    }
  free(fq);
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    if (!(in >> cmd)) continue;
    if (cmd == "call") std::cout << do_call(in) << "\n";
    else if (cmd == "quads") do_quads(in);
    else std::cout << "unknown command\n";
    std::cout.flush();
  }
  return 0;
}
