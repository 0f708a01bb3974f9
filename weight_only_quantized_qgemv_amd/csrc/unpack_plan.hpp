// unpack_plan.hpp — compile-time plan for turning a unit of 32 packed codes
// into pairs of 16-bit floats that a dot2 instruction consumes directly.
//
// Layout being unpacked (emily lib/emily/quantization.ex, `dequantize_defn/1`
// docs): lane i of a row sits at bit offset i*bits of the row's little-endian
// u32 stream. A unit of 32 consecutive codes occupies exactly `bits` words,
// starts on a word boundary and never shares a word with another unit.
//
// Trick: OR-ing a code q, shifted left by o, into the mantissa of the 16-bit
// float M = 2^e gives exactly M + q * 2^o, as long as the code's bits stay
// inside the mantissa (o + bits <= 7 for bf16 with M = 128, <= 10 for fp16
// with M = 1024). One v_and_or_b32 on a 32-bit window of the stream therefore
// produces two such values (low and high half) at once; the plan picks the
// windows (bit positions in the unit; a window that is not word aligned costs
// one v_alignbit_b32) and, for each pair, which code lands in each half and at
// which offset. The activation pair that meets it is pre-scaled by 2^-o, and
// the constant M * sum(x * 2^-o) is subtracted once per unit.
#pragma once

namespace qp {

struct PlanPair {
    int win;          // index of the window it reads
    int lo, hi;       // code index (0..31) in the low / high half, -1 if unused
    int lo_off, hi_off; // bit offset of the code inside its 16-bit half
};

struct UnpackPlan {
    bool feasible;
    int n_win;
    int win_bit[32];  // window start bit inside the unit (0 .. 32*bits - 1)
    int n_pair;
    PlanPair pair[32];
};

// Greedy cover: take the first uncovered code, try every window start that
// keeps it in the low half, keep the start that forms the most full pairs.
constexpr UnpackPlan make_unpack_plan(int bits, int mant)
{
    UnpackPlan p{};
    p.feasible = bits <= mant;
    if (!p.feasible)
        return p;
    bool covered[32] = {};
    for (int guard = 0; guard < 32; ++guard) {
        int c0 = -1;
        for (int c = 0; c < 32; ++c)
            if (!covered[c]) { c0 = c; break; }
        if (c0 < 0)
            break;
        int best_wb = -1, best_pairs = -1, best_codes = -1, best_aligned = 0;
        // c0 must sit in the low half: wb <= c0*bits and c0*bits + bits <= wb + mant.
        int lo0 = c0 * bits + bits - mant > 0 ? c0 * bits + bits - mant : 0;
        for (int wb = lo0; wb <= c0 * bits; ++wb) {
            int nl = 0, nh = 0;
            for (int c = 0; c < 32; ++c) {
                if (covered[c]) continue;
                int cb = c * bits;
                if (wb <= cb && cb + bits <= wb + mant) ++nl;
                else if (wb + 16 <= cb && cb + bits <= wb + 16 + mant) ++nh;
            }
            int np = nl < nh ? nl : nh;
            int aligned = (wb % 32) == 0;
            if (np > best_pairs || (np == best_pairs && nl + nh > best_codes) ||
                (np == best_pairs && nl + nh == best_codes && aligned > best_aligned)) {
                best_wb = wb; best_pairs = np; best_codes = nl + nh; best_aligned = aligned;
            }
        }
        int w = p.n_win++;
        p.win_bit[w] = best_wb;
        int L[16] = {}, H[16] = {}, nl = 0, nh = 0;
        for (int c = 0; c < 32; ++c) {
            if (covered[c]) continue;
            int cb = c * bits;
            if (best_wb <= cb && cb + bits <= best_wb + mant) L[nl++] = c;
            else if (best_wb + 16 <= cb && cb + bits <= best_wb + 16 + mant) H[nh++] = c;
        }
        int n = nl > nh ? nl : nh;
        for (int i = 0; i < n; ++i) {
            PlanPair& pp = p.pair[p.n_pair++];
            pp.win = w;
            pp.lo = i < nl ? L[i] : -1;
            pp.hi = i < nh ? H[i] : -1;
            pp.lo_off = i < nl ? L[i] * bits - best_wb : 0;
            pp.hi_off = i < nh ? H[i] * bits - best_wb - 16 : 0;
            if (pp.lo >= 0) covered[pp.lo] = true;
            if (pp.hi >= 0) covered[pp.hi] = true;
        }
    }
    return p;
}

} // namespace qp
