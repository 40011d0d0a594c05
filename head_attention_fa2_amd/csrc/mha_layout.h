// LDS tile layout of the attention kernel: 16-byte-chunk XOR swizzle, its inverse, and
// the operand-row permutation.  Plain integer functions usable on host and device so
// that the host test suite can check them exhaustively.
#ifndef MHA_LAYOUT_H_
#define MHA_LAYOUT_H_

#if defined(__HIPCC__)
#define MHA_HD __host__ __device__ __forceinline__
#else
#define MHA_HD inline
#endif

namespace mha_layout {

// Chunk permutation inside a 256-byte LDS line, for lines holding one row (sw16) or two
// rows (sw8).  sw8 puts line parity into bit 2: the transposing V^T read takes four
// consecutive keys (two lines, one even and one odd) x four chunks in one pass, and the two
// lines' chunks then fall into different halves of the bank groups.
MHA_HD constexpr int sw16(int x) { return ((x >> 2) & 3) | ((x & 3) << 2); }
MHA_HD constexpr int sw8(int x) { return ((x & 1) << 2) | ((x >> 1) & 3); }

// Byte offset in a K/V tile of 16-byte chunk c of row r, for rows of R chunks
// (R = 8: 128-byte rows, two per line; R = 16: one 256-byte line; R = 32: two lines).
template <int R>
MHA_HD constexpr int lds_off(int r, int c) {
  if constexpr (R == 8) {
    return (r >> 1) * 256 + (((((r & 1) << 3) | c) ^ sw8((r >> 1) & 7)) << 4);
  } else if constexpr (R == 16) {
    return r * 256 + ((c ^ sw16(r & 15)) << 4);
  } else {
    return r * 512 + (((c & 16) | ((c & 15) ^ sw16(r & 15))) << 4);
  }
}

// Inverse of lds_off: the (row, chunk) held by the 16-byte slot with linear index L.
template <int R>
MHA_HD constexpr void lds_inv(int L, int& r, int& c) {
  if constexpr (R == 8) {
    const int line = L >> 4;
    const int v = (L & 15) ^ sw8(line & 7);
    r = 2 * line + (v >> 3);
    c = v & 7;
  } else if constexpr (R == 16) {
    r = L >> 4;
    c = (L & 15) ^ sw16(r & 15);
  } else {
    r = L >> 5;
    c = (L & 16) | ((L & 15) ^ sw16(r & 15));
  }
}

// Row permutation inside a 32-row MFMA slab: swap bits 2 and 3.
MHA_HD constexpr int sigma(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// True when the swizzle phase repeats every kRowStep rows, so that load j of a thread
// reads chunk lds_inv(first slot) of row row0 + j*kRowStep.
template <int R>
MHA_HD constexpr bool loader_periodic() { return R == 8 || R == 16; }

// K operand (A operand of S^T = K.Q^T): lane (n = lane & 31, G = lane >> 5) at step kc
// reads 16 bytes: row sigma(n) of the first 32-row slab, chunk 2kc + G.  The second
// slab is 32 rows further.
template <int R>
MHA_HD constexpr int k_operand_off(int lane, int kc) {
  return lds_off<R>(sigma(lane & 31), 2 * kc + (lane >> 5));
}

// V^T operand (A operand of O^T = V^T.P^T, bf16, R = d/8 chunks per row) for output
// columns 32dt..32dt+31 and keys 0..15 of the tile, read with ds_read_b64_tr_b16 in two
// halves h = 0, 1 (keys 8G + 4h + 0..3).  In each 16-lane group the instruction returns
// to lane i, element e, sub-element i%4 of the 8 bytes addressed by lane 4e + i/4.
// Source lane s of group g16 therefore addresses key 8(g16 >> 1) + (s >> 2) + 4h and a
// 4-column group chosen so that output lane m receives column 32dt + sigma(m).
template <int R>
MHA_HD constexpr int v_operand_off(int lane, int dt, int h) {
  const int g16 = lane >> 4, s = lane & 15, a = s & 3;
  const int key = 8 * (g16 >> 1) + (s >> 2) + 4 * h;
  const int col = dt * 32 + 16 * (g16 & 1) + 4 * (a >> 1) + 8 * (a & 1);
  return lds_off<R>(key, col >> 3) + (col & 7) * 2;
}

}  // namespace mha_layout

#endif  // MHA_LAYOUT_H_
