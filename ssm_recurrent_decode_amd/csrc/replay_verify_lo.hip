// Instantiations of the ReplaySSM verify kernel for draft windows T = 1..4
// (own translation unit so the kernel variants compile in parallel).
#include "replay.hpp"

namespace rssm_host {

int launch_replay_verify_lo(int T, int D, const ReplayParams& p, int B, void* stream) {
  switch (T) {
    case 1: return D == 64 ? launch_window<64, 1, false>(p, B, stream) : launch_window<128, 1, false>(p, B, stream);
    case 2: return D == 64 ? launch_window<64, 2, false>(p, B, stream) : launch_window<128, 2, false>(p, B, stream);
    case 3: return D == 64 ? launch_window<64, 3, false>(p, B, stream) : launch_window<128, 3, false>(p, B, stream);
    case 4: return D == 64 ? launch_window<64, 4, false>(p, B, stream) : launch_window<128, 4, false>(p, B, stream);
    default: return RSSM_ENOTSUP;
  }
}

}  // namespace rssm_host
