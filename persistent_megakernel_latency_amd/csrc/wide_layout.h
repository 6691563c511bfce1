// wide_layout.h -- LDS layout of a wide (matrix-core) row block's reduction.
//
// The last K slice of a row block loads the other slices' partial sums into
// the operand area of its LDS (kWideFrags pieces of 1 KiB = 256 floats),
// together with what its epilogue reads: the RoPE factors of each sequence's
// position (q and k rows) and the RMSNorm sums of squares of the operand rows
// (the consumers of a normalised input: QKV, gate/up, LM head).  All of them
// are loaded in one round trip and read after the slice sums, so the slot
// pieces of every batch must stay clear of the RoPE and sums-of-squares
// pieces.  These functions are the single definition of that layout: the
// kernel computes its LDS offsets with them and the CPU tests enumerate every
// (slice count, own slice, sequence halves, operator) combination against
// them.  constexpr functions compile for the device as well as the host.
#pragma once
#include "plan.h"

namespace wpk {

constexpr int kWidePieces = (kWideK / 32) * 2 * 2;  // operand area: k-steps x sequence halves x hi/lo planes

// The kernel writes these expressions through the macros (so its code is
// exactly the expressions below); the constexpr functions wrap the same
// macros for the host-side checks.
#define WPK_WIDE_SLOT_PIECES(nh) (4 * (nh))
#define WPK_WIDE_FIT(nh) (16 / (nh))
#define WPK_WIDE_SS_PIECES(nrb) ((nrb) / 8)
#define WPK_WIDE_HAS_OWN(s0, c, fit) ((c) >= (s0) && (c) < (s0) + (fit) + 1)
#define WPK_WIDE_ADVANCE(s0, c, fit) ((c) >= (s0) && (c) < (s0) + (fit) + 1 ? 1 : 0)
#define WPK_WIDE_SLOT_OF(sl, s0, c, own) ((sl) - (s0) - ((sl) > (c) ? (own) : 0))
#define WPK_WIDE_ROPE_PIECE 48

// pieces of one partial-sum slot (64 rows x 16 sequences x 4 bytes per half)
constexpr int wide_slot_pieces(int nh) { return WPK_WIDE_SLOT_PIECES(nh); }
// partial-sum slots the operand area holds at once
constexpr int wide_fit(int nh) { return WPK_WIDE_FIT(nh); }
// RoPE factors of each sequence's position: cos in pieces [48, 52), sin in [52, 56)
constexpr int kWideRopePiece = WPK_WIDE_ROPE_PIECE;
constexpr int kWideRopePieces = 8;
// sums of squares [H / 64][32] floats, at the top of the area
constexpr int wide_ss_pieces(int hidden) { return WPK_WIDE_SS_PIECES(hidden / kWideRows); }
constexpr int wide_ss_first(int hidden) { return kWidePieces - wide_ss_pieces(hidden); }

// The slices of a row block are loaded in batches of at most wide_fit slots;
// the batch that holds the own slice c (which stays in the compute waves'
// partial-sum area and is not loaded) covers one slice more.  A batch starts
// at s0, the next at s0 + fit + wide_batch_has_own(s0, c, fit).
constexpr int wide_batch_has_own(int s0, int c, int fit) { return WPK_WIDE_ADVANCE(s0, c, fit); }
constexpr int wide_batch_end(int s0, int c, int fit, int nsl) {
  return nsl < s0 + fit + wide_batch_has_own(s0, c, fit) ? nsl : s0 + fit + wide_batch_has_own(s0, c, fit);
}
// the LDS slot of slice sl (sl != c) in the batch starting at s0
constexpr int wide_slot_of(int sl, int s0, int c, int has_own) { return WPK_WIDE_SLOT_OF(sl, s0, c, has_own); }

// Epilogue transposition area: [sequence][row] floats with pitch 68 from the
// start of the operand area (read after the slice sums are taken).
constexpr int kWideTransposePitch = 68;

}  // namespace wpk
