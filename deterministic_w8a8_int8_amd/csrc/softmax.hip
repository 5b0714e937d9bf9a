// Candidate softmax: the probabilities a decision read-out returns over its
// candidate tokens.
//
// The dsiab.com post on moving decision models from vLLM to Prism, section
// "方案", scores only the candidate tokens and normalises within that set;
// for a task with a fixed option set this equals the full-vocabulary
// softmax renormalised over the candidates.  The review page "StartLux-Prism:
// Fast, exact inference for StartLux-Decision models on NVIDIA GPUs" says
// the model returns probabilities for the available options and that the
// read-out path is fixed.  So the probabilities are computed here in one
// fixed sequence of binary64 operations, the same on every run and for any
// batch:
//   l_c   = (double) logit[m,c]                      (exact)
//   mx    = max_c l_c                                 (exact)
//   e_c   = exp64(l_c - mx)                           (see below)
//   S     = (((e_0 + e_1) + e_2) + ... ) + e_{C-1}    (candidate order)
//   p_c   = e_c / S                                   (IEEE division)
// A row holding a non-finite logit (the read-out writes a quiet NaN for an
// id outside the vocabulary) gets NaN for every candidate.
//
// exp64(z) for z <= 0: Cody and Waite's argument reduction (Cody & Waite,
// "Software Manual for the Elementary Functions", 1980) and a Taylor
// polynomial.
//   k = rint(z / ln 2),  r = (z - k*LN2_HI) - k*LN2_LO,  |r| <= ln2/2 + tiny
//   exp(r) ~ sum_{n=0..13} r^n / n!   (Horner, one fused multiply-add per
//   degree; truncation < 6e-18 relative)
//   exp64(z) = ldexp(exp(r), k)
// LN2_HI is ln 2 rounded to 37 significant bits, so k*LN2_HI is exact for
// |k| < 2^16, and z - k*LN2_HI is exact (Sterbenz); LN2_LO = ln 2 - LN2_HI
// rounded to binary64.  The coefficients are 1/n! rounded to binary64.  All
// were derived from an 80-digit ln 2 and exact rationals.  The relative error
// of exp64 is a few units in the last place; that of p_c at most about
// (C + 6) units in the last place.
#include "device_common.h"
#include "launch.h"
#include "softmax_row.h"

namespace w8a8 {

namespace {

// One wave per row; lane c holds candidate c (C <= 64).
__global__ __launch_bounds__(64) void candidate_softmax_kernel(const float* __restrict__ logits,
                                                               int64_t C, double* __restrict__ probs) {
    const int64_t m = blockIdx.x;
    const int c = threadIdx.x;
    const bool live = c < C;
    const float lf = live ? logits[m * C + c] : 0.0f;
    const double p = candidate_softmax_wave(lf, live, static_cast<int>(C));
    if (live) probs[m * C + c] = p;
}

}  // namespace

hipError_t launch_candidate_softmax(const float* logits, int64_t M, int64_t C, double* probs,
                                    hipStream_t stream) {
    if (M <= 0 || C <= 0) return hipSuccess;
    hipLaunchKernelGGL(candidate_softmax_kernel, dim3(static_cast<unsigned>(M)), dim3(64), 0, stream,
                       logits, C, probs);
    return hipGetLastError();
}

}  // namespace w8a8
