// Instantiations of the GDN verify kernel for draft windows T = 5..8
// (own translation unit so the kernel variants compile in parallel).
#include "gdn.hpp"

namespace rssm_host {

int launch_gdn_verify_hi(int T, int D, const GdnReplayParams& p, int B, void* stream) {
  switch (T) {
    case 5: return D == 64 ? launch_gdn_window<64, 5>(p, B, stream) : launch_gdn_window<128, 5>(p, B, stream);
    case 6: return D == 64 ? launch_gdn_window<64, 6>(p, B, stream) : launch_gdn_window<128, 6>(p, B, stream);
    case 7: return D == 64 ? launch_gdn_window<64, 7>(p, B, stream) : launch_gdn_window<128, 7>(p, B, stream);
    case 8: return D == 64 ? launch_gdn_window<64, 8>(p, B, stream) : launch_gdn_window<128, 8>(p, B, stream);
    default: return RSSM_ENOTSUP;
  }
}

}  // namespace rssm_host
