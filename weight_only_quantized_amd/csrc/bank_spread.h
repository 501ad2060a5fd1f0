// Host-side order within groups for act-order layers (called by gptq_repack); plain C++, so that
// a host build can check it (tests/spread_check.cpp).
#pragma once
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "layout.h"

namespace gq {

// Order within groups for the act-order staging of the skinny kernel.  The load-time sort only has
// to make every group contiguous ("39. Quantized checkpoints ...", section "GPTQ": inputs sorted by
// g_idx once at load time); a group shares one scale and one zero per output, so any order of its
// inputs gives the same sums.  That freedom is used here.  The kernel stages x through the inverse
// permutation: a lane loads 8 consecutive inputs and writes each to LDS at its sorted position, so
// one 2-byte write instruction of a wave covers the inputs 512 b + 8 L + e of one block b, lanes
// L = 0..63, one e = 0..7.  In the stable order those positions fall on random LDS banks (measured
// on MI355X: about 13 conflict cycles per write instruction).  Here each input instead takes a
// position in its group whose bank (4-byte word mod 64) differs from every other lane's of the same
// instruction, with distinct banks mod 32 within each half-wave as well.
//
// Construction: a bipartite multigraph with one edge per input (padding inputs past K join a
// padding group) between its half-instruction (block, e, lane / 32: 32 edges) and its group (a
// multiple of 128 edges).  Five Euler splits (edges alternate along closed trails, so every node
// keeps half its edges on each side) give 32 classes with one edge per half-instruction: the bank
// mod 32.  A sixth split with the two halves of an instruction as one node (two edges per class)
// gives bit 5.  Each group then holds every bank exactly size / 64 times, which is how often its
// 128-aligned positions use each bank.  Applies when every group is a multiple of 128 inputs and
// x fits the staging (Kp <= 8192); returns false, leaving perm alone, otherwise.
inline void euler_split(int n_nodes, const std::vector<int>& a, const std::vector<int>& b,
                        const std::vector<int>& edges, std::vector<uint8_t>& label) {
  // CSR adjacency over the edges of this class (endpoints a[e] and b[e], b offset past the a-nodes)
  std::vector<int> start(n_nodes + 1, 0), adj(2 * edges.size()), ptr;
  for (int e : edges) { start[a[e] + 1]++; start[b[e] + 1]++; }
  for (int v = 0; v < n_nodes; ++v) start[v + 1] += start[v];
  ptr.assign(start.begin(), start.end() - 1);
  for (int e : edges) { adj[ptr[a[e]]++] = e; adj[ptr[b[e]]++] = e; }
  ptr.assign(start.begin(), start.end() - 1);
  std::vector<uint8_t> used(a.size(), 0);
  for (int v0 = 0; v0 < n_nodes; ++v0) {
    for (;;) {
      while (ptr[v0] < start[v0 + 1] && used[adj[ptr[v0]]]) ptr[v0]++;
      if (ptr[v0] == start[v0 + 1]) break;
      int v = v0;
      uint8_t side = 0;
      for (;;) {   // a closed trail from v0 (every degree is even), labels alternating
        while (ptr[v] < start[v + 1] && used[adj[ptr[v]]]) ptr[v]++;
        if (ptr[v] == start[v + 1]) break;
        const int e = adj[ptr[v]];
        used[e] = 1;
        label[e] = side;
        side ^= 1;
        v = a[e] == v ? b[e] : a[e];
      }
    }
  }
}

inline bool spread_scatter_banks(int K, int Kp, int gs_eff, int32_t* perm) {
  if (Kp > kIpermMaxKp || K % 128 != 0 || gs_eff % 128 != 0) return false;
  const int NB = (K + 511) / 512, NS = NB * 512, G = (K + gs_eff - 1) / gs_eff;
  std::vector<int> group_of(NS);
  for (int j = 0; j < K; ++j) group_of[perm[j]] = j / gs_eff;
  for (int k = K; k < NS; ++k) group_of[k] = G;                 // padding group (a multiple of 128)
  const int NH = NB * 16;                                       // half-instructions
  std::vector<int> a(NS), bn(NS);
  for (int k = 0; k < NS; ++k) {
    const int blk = k >> 9, lane = (k >> 3) & 63, e = k & 7;
    a[k] = (blk * 8 + e) * 2 + (lane >> 5);
    bn[k] = NH + group_of[k];
  }
  std::vector<int> color(NS, 0);
  std::vector<uint8_t> label(NS, 0);
  std::vector<std::vector<int>> classes(1);
  classes[0].resize(NS);
  for (int k = 0; k < NS; ++k) classes[0][k] = k;
  for (int level = 0; level < 6; ++level) {
    if (level == 5)
      for (int k = 0; k < NS; ++k) a[k] >>= 1;                  // the two halves of an instruction as one node
    std::vector<std::vector<int>> next;
    for (auto& cl : classes) {
      euler_split(NH + G + 1, a, bn, cl, label);
      std::vector<int> c0, c1;
      for (int k : cl) (label[k] ? c1 : c0).push_back(k);
      for (int k : c1) color[k] |= level < 5 ? (1 << level) : 32;
      next.push_back(std::move(c0));
      next.push_back(std::move(c1));
    }
    classes.swap(next);
  }
  // positions of each group by bank, inputs of each colour in ascending order
  std::vector<int32_t> out(K, -1);
  std::vector<int> fill((size_t)G * 64, 0);
  for (int k = 0; k < K; ++k) {
    const int g = group_of[k], c = color[k];
    const int i = fill[(size_t)g * 64 + c]++;                  // i-th position of bank c in group g
    const int q = (i >> 1) * 128 + 2 * c + (i & 1);
    if (q >= std::min(gs_eff, K - g * gs_eff)) return false;
    out[g * gs_eff + q] = k;
  }
  // check before use: a permutation, groups unchanged, banks distinct per instruction and half-wave
  std::vector<uint8_t> seen(K, 0);
  std::vector<int> pos(K);
  for (int j = 0; j < K; ++j) {
    if (out[j] < 0 || seen[out[j]] || group_of[out[j]] != j / gs_eff) return false;
    seen[out[j]] = 1;
    pos[out[j]] = j;
  }
  for (int blk = 0; blk < NB; ++blk)
    for (int e = 0; e < 8; ++e) {
      uint64_t banks = 0;
      uint32_t half[2] = {0u, 0u};
      for (int lane = 0; lane < 64; ++lane) {
        const int k = blk * 512 + lane * 8 + e;
        if (k >= K) continue;
        const int bank = (pos[k] >> 1) & 63;
        if ((banks >> bank) & 1 || (half[lane >> 5] >> (bank & 31)) & 1) return false;
        banks |= 1ull << bank;
        half[lane >> 5] |= 1u << (bank & 31);
      }
    }
  memcpy(perm, out.data(), sizeof(int32_t) * K);
  return true;
}

}  // namespace gq
