// Encoder instantiations for a bit budget of 5 bits per coordinate.
#include "k_encode_kernels.hpp"

namespace octo {

hipError_t launch_encode_b5(int d, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                            int64_t n_seq, hipStream_t s) {
  return launch_encode_b<5>(d, kdt, qjl, joint, a, n_seq, s);
}

}  // namespace octo
