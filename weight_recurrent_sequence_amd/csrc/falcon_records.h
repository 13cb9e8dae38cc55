// falcon_records.h -- the per-tile workspace record the intra-chunk kernel
// writes and the state passes (forward and backward) read.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace falcon {

// Record of one (batch*head, tile) of CV virtual rows, element type E:
//   -A, its strictly lower 16 x 16 blocks (delta family);
//   (I + A_bb)^-1, the inverses of the diagonal blocks (delta family);
//   P, its blocks on and below the diagonal (with a window: the blocks of
//   the first two query blocks, row-major);
// each block in MFMA fragment order (64 lanes x 4 values: lane (lr, grp)
// holds M[lr][4 grp + r]); then five arrays of CV floats: gam = exp(g of the
// row's step), hrow = exp(g_last - g of the row's step) times the row's write
// scale, gq = exp(g_t), l1 = ||x_i||_1, erow = eta of the row's step.
template <class E, int CV, bool DELTA>
struct Rec {
    static constexpr int NB = CV / 16;
    static constexpr int NBA = DELTA ? NB * (NB - 1) / 2 : 0;  // strictly lower blocks of -A
    static constexpr int NBD = DELTA ? NB : 0;                 // (I + A_bb)^-1
    static constexpr int NBP = NB * NB;                        // blocks of P
    static constexpr size_t kA = 0;                            // element offsets
    static constexpr size_t kD = (size_t)NBA * 256;
    static constexpr size_t kP = (size_t)(NBA + NBD) * 256;
    static constexpr size_t kScalBytes = (size_t)(NBA + NBD + NBP) * 256 * E::kBytes;
    static constexpr int NSC = 5;  // gam, hrow, gq, l1, erow (CV floats each)
    static constexpr size_t kBytes = (kScalBytes + NSC * CV * 4 + 255) / 256 * 256;
    static __host__ __device__ constexpr int ablk(int b, int c) { return b * (b - 1) / 2 + c; }
    // P block (b, c): without a window the blocks on and below the diagonal in
    // row order; with one (two query blocks at most) row-major over them.
    static __host__ __device__ constexpr int pblk(int b, int c, bool win) {
        return win ? b * NB + c : b * (b + 1) / 2 + c;
    }
    static constexpr int npblk(bool win) { return win ? 2 * NB : NB * (NB + 1) / 2; }
};

__host__ __device__ inline int tiles_of(int T, int Ct) { return (T + Ct - 1) / Ct; }

}  // namespace falcon
