// Bounds check of the LDS layout a wide row block's last slice uses for its
// reduction (wide_layout.h, the functions the kernel computes its offsets
// with), over every slice count, own slice, number of 16-sequence halves and
// operator the builder can emit.  Prints one line per violation and exits
// nonzero if there is any.
#include <cstdio>
#include <vector>

#include "wide_layout.h"

using namespace wpk;

static int failures = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      ++failures;                        \
      if (failures < 50) {               \
        std::printf(__VA_ARGS__);        \
        std::printf("\n");               \
      }                                  \
    }                                    \
  } while (0)

int main() {
  constexpr int kOperandFloats = kWidePieces * 256;
  constexpr int kLdsFloats = kOperandFloats + kWidePart;  // the kernel's wide LDS area
  static_assert(kWidePart == 8 * 256, "own partial sums: 8 pieces after the operand area");
  long combos = 0;
  for (int hidden = 512; hidden <= 2048; hidden += 512) {
    for (int ffn = 512; ffn <= 16384; ffn += 512) {
      for (int nh = 1; nh <= 2; ++nh) {
        // operators: 0 qkv q/k rows (RoPE), 1 qkv v rows, 2 o-proj, 3 gate/up, 4 down, 5 LM head
        for (int op = 0; op <= 5; ++op) {
          const int K = op == 4 ? ffn : hidden;
          const int nsl = K / kWideK;
          const bool consumer = op == 0 || op == 1 || op == 3 || op == 5;
          const bool rope = op == 0;
          const int per = wide_slot_pieces(nh), fit = wide_fit(nh);
          CHECK(fit >= 1 && fit * per <= kWidePieces, "fit %d per %d", fit, per);
          const int ss0 = wide_ss_first(hidden), ss1 = kWidePieces;
          CHECK(ss0 >= 0 && ss0 < ss1, "sums of squares pieces [%d, %d) for hidden %d", ss0, ss1, hidden);
          if (consumer) CHECK(!rope || ss0 >= kWideRopePiece + kWideRopePieces, "RoPE and sums of squares overlap");
          for (int c = 0; c < nsl; ++c) {
            ++combos;
            std::vector<int> loaded(nsl, 0);
            int batches = 0;
            for (int s0 = 0; s0 < nsl; s0 += fit + wide_batch_has_own(s0, c, fit)) {
              CHECK(++batches <= nsl, "batch loop does not advance (nsl %d c %d nh %d)", nsl, c, nh);
              if (batches > nsl) break;
              const int own = wide_batch_has_own(s0, c, fit);
              const int s1 = wide_batch_end(s0, c, fit, nsl);
              CHECK(s1 > s0 && s1 <= nsl, "batch [%d, %d) of %d slices", s0, s1, nsl);
              std::vector<int> used(fit, 0);
              for (int sl = s0; sl < s1; ++sl) {
                if (sl == c) continue;
                const int slot = wide_slot_of(sl, s0, c, own);
                CHECK(slot >= 0 && slot < fit, "slot %d of slice %d outside [0, %d) (nsl %d c %d nh %d)", slot, sl,
                      fit, nsl, c, nh);
                if (slot < 0 || slot >= fit) continue;
                CHECK(!used[slot], "slot %d used twice in batch %d (nsl %d c %d nh %d)", slot, s0, nsl, c, nh);
                used[slot] = 1;
                loaded[sl]++;
                const int p0 = slot * per, p1 = p0 + per;  // pieces the slice's partial sums land in
                CHECK(p1 <= kWidePieces, "slot pieces [%d, %d) past the operand area", p0, p1);
                if (rope)
                  CHECK(p1 <= kWideRopePiece || p0 >= kWideRopePiece + kWideRopePieces,
                        "slot pieces [%d, %d) overlap the RoPE factors (op %d nsl %d c %d nh %d)", p0, p1, op, nsl, c,
                        nh);
                if (consumer)
                  CHECK(p1 <= ss0, "slot pieces [%d, %d) overlap the sums of squares [%d, %d) (op %d nsl %d c %d)", p0,
                        p1, ss0, ss1, op, nsl, c);
              }
            }
            for (int sl = 0; sl < nsl; ++sl)
              CHECK(loaded[sl] == (sl == c ? 0 : 1), "slice %d loaded %d times (nsl %d c %d nh %d)", sl, loaded[sl],
                    nsl, c, nh);
          }
          // the epilogue's transposition rows: 32 sequences x pitch, written after
          // the slice sums, read with the RoPE factors
          const int tr_floats = 32 * kWideTransposePitch;
          CHECK(tr_floats <= kOperandFloats, "transposition area past the operand area");
          if (rope) CHECK(tr_floats <= kWideRopePiece * 256, "transposition area overlaps the RoPE factors");
          // the RoPE reads: rl[n * 32 + d] and rl[1024 + n * 32 + d] for n, d < 32
          if (rope) CHECK(kWideRopePiece * 256 + 2048 <= kWideRopePiece * 256 + kWideRopePieces * 256, "RoPE extent");
          // the compute waves' partial sums: [half][row][16 sequences] after the operand area
          CHECK(kOperandFloats + (nh * kWideRows) * 16 <= kLdsFloats, "own partial sums past the LDS area");
        }
      }
    }
  }
  std::printf("wide layout: %ld combinations, %d violations\n", combos, failures);
  return failures ? 1 : 0;
}
