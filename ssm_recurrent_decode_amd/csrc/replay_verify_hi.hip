// Instantiations of the ReplaySSM verify kernel for draft windows T = 5..8
// (own translation unit so the kernel variants compile in parallel).
#include "replay.hpp"

namespace rssm_host {

int launch_replay_verify_hi(int T, int D, const ReplayParams& p, int B, void* stream) {
  switch (T) {
    case 5: return D == 64 ? launch_window<64, 5, false>(p, B, stream) : launch_window<128, 5, false>(p, B, stream);
    case 6: return D == 64 ? launch_window<64, 6, false>(p, B, stream) : launch_window<128, 6, false>(p, B, stream);
    case 7: return D == 64 ? launch_window<64, 7, false>(p, B, stream) : launch_window<128, 7, false>(p, B, stream);
    case 8: return D == 64 ? launch_window<64, 8, false>(p, B, stream) : launch_window<128, 8, false>(p, B, stream);
    default: return RSSM_ENOTSUP;
  }
}

}  // namespace rssm_host
