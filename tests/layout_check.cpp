// Host check of the kernel's LDS layout and operand addressing (mha_layout.h):
//  1. lds_off / lds_inv are inverse bijections on a 64-row tile;
//  2. the tile loader (4 wavefronts x 64 lanes x kLoads 16-byte copies) writes every
//     (row, chunk) of the tile exactly once, at the slot lds_off says;
//  3. the K operand of every lane and step is row sigma(n) (+32 per slab), chunk 2kc+G;
//  4. the V^T operand built by two ds_read_b64_tr_b16 per MFMA is, on lane L element e,
//     V[16 kc2 + 8G + e][32 dt + sigma(L & 31)] (bf16 tiles);
//  5. bank use: each 16-lane pass of the K read (ds_read_b128) touches distinct 16-byte
//     bank groups, and each 32-lane pass of a V^T read (ds_read_b64_tr_b16) asks no
//     four-byte bank for two different words (printed as counts of conflicts).
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "mha_layout.h"

using namespace mha_layout;
static int failures = 0;
#define CHECK(c, ...) do { if (!(c)) { if (failures++ < 20) { printf("FAIL %s:%d ", __FILE__, __LINE__); printf(__VA_ARGS__); printf("\n"); } } } while (0)

template <int R>
void check(int elem_bytes) {
  const int RB = R * 16, tile = 64 * RB, waves = 4, loads = 64 * R / (waves * 64);
  const int d = RB / elem_bytes;
  // 1. bijection
  std::vector<int> seen(tile / 16, 0);
  for (int r = 0; r < 64; ++r)
    for (int c = 0; c < R; ++c) {
      const int off = lds_off<R>(r, c);
      CHECK(off % 16 == 0 && off >= 0 && off < tile, "R=%d off range", R);
      seen[off / 16]++;
      int r2, c2;
      lds_inv<R>(off / 16, r2, c2);
      CHECK(r2 == r && c2 == c, "R=%d inverse r=%d c=%d", R, r, c);
    }
  for (int x : seen) CHECK(x == 1, "R=%d not a bijection", R);
  // 2. loader (the kernel's formulas: periodic shortcut or per-load inverse)
  std::vector<int> loaded(64 * R, 0);
  const int row_step = 1024 * waves / RB;
  for (int w = 0; w < waves; ++w)
    for (int lane = 0; lane < 64; ++lane) {
      int r0, c0;
      lds_inv<R>(w * 64 + lane, r0, c0);
      for (int j = 0; j < loads; ++j) {
        int r, c;
        if (loader_periodic<R>() && j > 0) { r = r0 + j * row_step; c = c0; }
        else lds_inv<R>((j * waves + w) * 64 + lane, r, c);
        const int slot = ((j * waves + w) * 1024 + lane * 16) / 16;
        int rt, ct;
        lds_inv<R>(slot, rt, ct);
        CHECK(r == rt && c == ct, "R=%d loader w=%d lane=%d j=%d", R, w, lane, j);
        CHECK(r >= 0 && r < 64 && c >= 0 && c < R, "R=%d loader range", R);
        loaded[r * R + c]++;
      }
    }
  for (int x : loaded) CHECK(x == 1, "R=%d loader coverage", R);
  // 3. K operand (bf16: 8 per chunk; fp32: 4 per chunk -> same chunk rule)
  const int ksteps = d / (elem_bytes == 2 ? 16 : 8);
  int kconf = 0;
  for (int kc = 0; kc < ksteps; ++kc) {
    for (int lane = 0; lane < 64; ++lane) {
      int r, c;
      lds_inv<R>(k_operand_off<R>(lane, kc) / 16, r, c);
      CHECK(r == sigma(lane & 31) && c == 2 * kc + (lane >> 5), "R=%d K operand", R);
    }
    for (int g = 0; g < 4; ++g) {   // 16-lane groups of ds_read_b128
      int used[16] = {0};
      for (int l = 16 * g; l < 16 * g + 16; ++l) used[(k_operand_off<R>(l, kc) / 16) % 16]++;
      for (int u : used) kconf += u > 1;
    }
  }
  // 4/5. V^T operand via the transposing read (bf16 only)
  int vconf = 0;
  if (elem_bytes == 2) {
    for (int dt = 0; dt < d / 32; ++dt)
      for (int kc2 = 0; kc2 < 4; ++kc2)
        for (int h = 0; h < 2; ++h) {
          for (int L = 0; L < 64; ++L) {
            const int g16 = L >> 4, i = L & 15;
            for (int e = 0; e < 4; ++e) {
              const int src = 16 * g16 + 4 * e + i / 4;
              const int byte = v_operand_off<R>(src, dt, h) + kc2 * 16 * RB + 2 * (i % 4);
              int r, c;
              lds_inv<R>(byte / 16, r, c);
              const int col = c * 8 + (byte % 16) / 2;
              const int G = L >> 5;
              CHECK(r == 16 * kc2 + 8 * G + 4 * h + e, "R=%d V key L=%d e=%d", R, L, e);
              CHECK(col == 32 * dt + sigma(L & 31), "R=%d V col L=%d e=%d", R, L, e);
            }
          }
          // 32 lanes (256 bytes) per pass from 64 four-byte banks: a pass is free of
          // conflicts when no bank is asked for two different words
          for (int g = 0; g < 2; ++g) {
            int word_of_bank[64];
            for (int b = 0; b < 64; ++b) word_of_bank[b] = -1;
            for (int l = 32 * g; l < 32 * g + 32; ++l)
              for (int w = 0; w < 2; ++w) {
                const int word = (v_operand_off<R>(l, dt, h) + kc2 * 16 * RB) / 4 + w;
                int& slot = word_of_bank[word % 64];
                if (slot >= 0 && slot != word) ++vconf;
                slot = word;
              }
          }
        }
  }
  printf("R=%d elem=%d: K-read conflicting bank groups %d, V-read conflicting bank groups %d\n",
         R, elem_bytes, kconf, vconf);
}

int main() {
  check<8>(2);    // bf16 d=64
  check<16>(2);   // bf16 d=128
  check<16>(4);   // fp32 d=64
  check<32>(4);   // fp32 d=128
  check<32>(2);   // 16-bit rows of 512 bytes: the GEMM's 256-column B tile, read as B^T
  printf(failures ? "layout check FAILED (%d)\n" : "layout check ok\n", failures);
  return failures ? 1 : 0;
}
