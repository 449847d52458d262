// headwise.hip -- head-wise tied dynamic short convolution, forward and
// backward, for gfx950 ("Dynamic Short Convolutions Improve Transformers",
// gist.science technical summary, Methodology: mechanism, parametrization (2)
// head-wise tying, placement with residual).  The kernels, their design and
// the launch rules are in headwise_impl.h; this file instantiates the layer
// alone.
#include "headwise_impl.h"

namespace dsc {

// A chunk holds whole groups (H divides VEC), or a group spans H / VEC
// chunks on at most 64 lanes (rounded up to a power of two in the backward).
bool headwise_fast(Dtype dt, int32_t H) {
    const int VEC = dt == Dtype::BF16 ? BF16::kVec : F32::kVec;
    if (H < 1) return false;
    if (H < VEC) return VEC % H == 0;
    return H % VEC == 0 && H / VEC <= kWave;
}

hipError_t headwise_fwd(const HwProblem &p, hipStream_t s) {
    if (!headwise_fast(p.dtype, p.H)) return headwise_any(p, s, false, false);
    return p.dtype == Dtype::BF16 ? dispatch<BF16, false>(p, s, false) : dispatch<F32, false>(p, s, false);
}

hipError_t headwise_bwd(const HwProblem &p, hipStream_t s) {
    if (!headwise_fast(p.dtype, p.H)) return headwise_any(p, s, true, false);
    return p.dtype == Dtype::BF16 ? dispatch<BF16, false>(p, s, true) : dispatch<F32, false>(p, s, true);
}

}  // namespace dsc
