// OCTOPUS online key encoder for gfx950: launch routing by bit budget.  The
// kernels are in k_encode_kernels.hpp; each bit budget's instantiations are
// compiled in k_encode_b<N>.hip.
#include "k_encode_kernels.hpp"

namespace octo {

hipError_t launch_encode_b1(int d, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                            int64_t n_seq, hipStream_t s);
hipError_t launch_encode_b2(int d, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                            int64_t n_seq, hipStream_t s);
hipError_t launch_encode_b3(int d, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                            int64_t n_seq, hipStream_t s);
hipError_t launch_encode_b4(int d, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                            int64_t n_seq, hipStream_t s);
hipError_t launch_encode_b5(int d, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                            int64_t n_seq, hipStream_t s);

hipError_t launch_encode(int d, int b, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                         int64_t n_seq, hipStream_t s) {
  if (a.n_new <= 0 || n_seq <= 0) return hipSuccess;
  switch (b) {
    case 1: return launch_encode_b1(d, kdt, qjl, joint, a, n_seq, s);
    case 2: return launch_encode_b2(d, kdt, qjl, joint, a, n_seq, s);
    case 3: return launch_encode_b3(d, kdt, qjl, joint, a, n_seq, s);
    case 4: return launch_encode_b4(d, kdt, qjl, joint, a, n_seq, s);
    case 5: return launch_encode_b5(d, kdt, qjl, joint, a, n_seq, s);
  }
  return hipErrorInvalidValue;
}

int lds_copies_encode(LdsCopyRec* out, int max) {
  int n = 0;
  n = enc_copy_recs_b<1>(out, n, max);
  n = enc_copy_recs_b<2>(out, n, max);
  n = enc_copy_recs_b<3>(out, n, max);
  n = enc_copy_recs_b<4>(out, n, max);
  n = enc_copy_recs_b<5>(out, n, max);
  return n;
}

}  // namespace octo
