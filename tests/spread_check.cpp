// Host check of the within-group order of act-order layers (weight_only_quantized_amd/csrc/
// bank_spread.h).  For seeded act-order group maps over K = 128 .. 8192 and groups of 128, 256, 512
// inputs and one group of all K, the stable group sort followed by spread_scatter_banks must
// succeed and give, checked here independently of the function's own check: a permutation of the
// inputs, every group's inputs on its own sorted positions, and for every 2-byte LDS write
// instruction of the staging (inputs 512 b + 8 L + e, lanes L = 0..63) 64 distinct banks (4-byte
// word of the sorted position mod 64) and 32 distinct banks mod 32 in each half of the wave.
// Shapes outside its reach (K not a multiple of 128, more than 8192 inputs) must leave the order
// alone.  Built with g++ by tests/test_boundary_cpu.py; prints "ok" on success.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "bank_spread.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32() {   // splitmix64
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

// g[k] = perm(k) / gs for a random permutation (act-order), then the stable sort by group
static std::vector<int32_t> sorted_order(int K, int gs, std::vector<int>& g) {
  std::vector<int> p(K);
  for (int k = 0; k < K; ++k) p[k] = k;
  for (int k = K - 1; k > 0; --k) std::swap(p[k], p[next_u32() % (uint32_t)(k + 1)]);
  g.assign(K, 0);
  for (int k = 0; k < K; ++k) g[k] = p[k] / gs;
  const int G = (K + gs - 1) / gs;
  std::vector<int> start(G + 1, 0);
  for (int k = 0; k < K; ++k) start[g[k] + 1]++;
  for (int q = 0; q < G; ++q) start[q + 1] += start[q];
  std::vector<int32_t> perm(K);
  for (int k = 0; k < K; ++k) perm[start[g[k]]++] = k;
  return perm;
}

static int check(int K, int gs) {
  std::vector<int> g;
  std::vector<int32_t> perm = sorted_order(K, gs, g);
  if (!gq::spread_scatter_banks(K, K, gs, perm.data())) { printf("refused K=%d gs=%d\n", K, gs); return 1; }
  std::vector<int> pos(K, -1);
  for (int j = 0; j < K; ++j) {
    const int k = perm[j];
    if (k < 0 || k >= K || pos[k] != -1) { printf("not a permutation K=%d gs=%d\n", K, gs); return 1; }
    if (g[k] != j / gs) { printf("group moved K=%d gs=%d\n", K, gs); return 1; }
    pos[k] = j;
  }
  for (int b = 0; b * 512 < K; ++b)
    for (int e = 0; e < 8; ++e) {
      uint64_t all = 0;
      uint32_t half[2] = {0, 0};
      for (int lane = 0; lane < 64; ++lane) {
        const int k = b * 512 + lane * 8 + e;
        if (k >= K) continue;
        const int bank = (pos[k] / 2) % 64;
        if (((all >> bank) & 1) || ((half[lane / 32] >> (bank % 32)) & 1)) {
          printf("bank conflict K=%d gs=%d block=%d e=%d\n", K, gs, b, e);
          return 1;
        }
        all |= 1ull << bank;
        half[lane / 32] |= 1u << (bank % 32);
      }
    }
  return 0;
}

int main() {
  int n = 0;
  for (int K = 128; K <= 8192; K += 128)
    for (int gs : {128, 256, 512, -1}) {
      const int ge = gs == -1 ? K : gs;
      if (ge > K || K % ge != 0) continue;
      for (int rep = 0; rep < (K == 8192 ? 8 : 1); ++rep) {
        if (check(K, ge)) return 1;
        ++n;
      }
    }
  // outside its reach: the order is left as it is
  for (int K : {1056, 8320}) {
    std::vector<int> g;
    std::vector<int32_t> perm = sorted_order(K, 32, g), keep = perm;
    if (gq::spread_scatter_banks(K, (K + 127) / 128 * 128, 32, perm.data()) || perm != keep) {
      printf("changed an order it cannot spread K=%d\n", K);
      return 1;
    }
  }
  if (n < 100) { printf("too few cases %d\n", n); return 1; }
  printf("ok\n");
  return 0;
}
